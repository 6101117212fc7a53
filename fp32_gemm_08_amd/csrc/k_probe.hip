// Matrix-core ceiling probe: the FP32 MFMA rate the chip sustains with no
// memory traffic, and the shader clock it runs at.
//
// The FP32 roofline of the GEMM is the matrix cores' rate; its published
// figure assumes every SIMD issues one v_mfma_f32_32x32x2_f32 per 64 cycles at
// 2.4 GHz.  This kernel measures what the part actually sustains: each
// wavefront runs a chain of such MFMAs on four independent accumulators (so
// no MFMA waits for the previous one's result) with random operands that
// differ from one MFMA to the next (eight operand pairs in rotation, as a
// GEMM's operand stream toggles the inputs), and nothing else.  Wavefront 0 of
// each workgroup reads the shader cycle counter (s_memtime) and the constant
// 100 MHz counter (s_memrealtime) around its chain; their ratio is the shader
// clock over the run.  Only vector stores write memory.
//
// Beside it, two more probes for the other ceilings of the MFMA kernels:
//  * the same chain on the 16-bit matrix cores (v_mfma_f32_32x32x16_{f16,bf16},
//    32768 FLOP each), with random or all-zero operands: the published 16-bit
//    rate assumes the full clock, and the clock the part holds under a 16-bit
//    matrix-core load depends on how much the operands toggle;
//  * the direct global->LDS load stream alone (global_load_lds_dwordx4, 1 KB
//    per wavefront instruction, the staging of the MFMA kernels): bytes per
//    shader cycle one CU takes in from L2 / the Infinity Cache / HBM, by the
//    number of wavefronts and of loads each keeps in flight.
#include "probe_internal.h"
#include "lp_types.h"

namespace sgemm {

namespace {

typedef float probe_f32x16 __attribute__((ext_vector_type(16)));

__device__ inline probe_f32x16 probe_mma(float a, float b, probe_f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// An integer mix (xorshift-multiply) mapped to a float in [-1, 1).
__device__ inline float probe_rand(unsigned x)
{
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return __uint_as_float((x >> 9) | 0x40000000U) - 3.0f;
}

__device__ inline unsigned long long probe_shader_cycles() { return __builtin_amdgcn_s_memtime(); }
__device__ inline unsigned long long probe_ref_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// trips: loop trips per wavefront, each issuing 8 MFMAs (two on each
// accumulator).  sink: one float per work-item; clocks: two counters per
// workgroup (shader cycles, then 100 MHz ticks).
__global__ __launch_bounds__(256) void mfma_probe_kernel(int trips, float *__restrict__ sink,
                                                          unsigned long long *__restrict__ clocks)
{
    const unsigned id = blockIdx.x * 256u + threadIdx.x;
    float a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = probe_rand(id * 16u + j);
        b[j] = probe_rand(id * 16u + 8u + j);
    }
    probe_f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const unsigned long long t0 = probe_shader_cycles(), r0 = probe_ref_ticks();
    for (int i = 0; i < trips; ++i) {
        c0 = probe_mma(a[0], b[0], c0);
        c1 = probe_mma(a[1], b[1], c1);
        c2 = probe_mma(a[2], b[2], c2);
        c3 = probe_mma(a[3], b[3], c3);
        c0 = probe_mma(a[4], b[4], c0);
        c1 = probe_mma(a[5], b[5], c1);
        c2 = probe_mma(a[6], b[6], c2);
        c3 = probe_mma(a[7], b[7], c3);
    }
    const unsigned long long t1 = probe_shader_cycles(), r1 = probe_ref_ticks();
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
    sink[id] = s;
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// 16-bit chain: as mfma_probe_kernel, eight operand pairs of 8 values per
// lane (random in [-1, 1), or all zero) rotating over four accumulators.
template <bool BF16>
__global__ __launch_bounds__(256) void mfma_lp_probe_kernel(int trips, int zero, float *__restrict__ sink,
                                                             unsigned long long *__restrict__ clocks)
{
    typedef typename Lp<BF16>::T T;
    typedef typename Lp<BF16>::V8 V8;
    const unsigned id = blockIdx.x * 256u + threadIdx.x;
    V8 a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            a[j][q] = (T)(zero ? 0.0f : probe_rand(id * 128u + 8u * j + q));
            b[j][q] = (T)(zero ? 0.0f : probe_rand(id * 128u + 64u + 8u * j + q));
        }
    lp_f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const unsigned long long t0 = probe_shader_cycles(), r0 = probe_ref_ticks();
    for (int i = 0; i < trips; ++i) {
        c0 = Lp<BF16>::mma(a[0], b[0], c0);
        c1 = Lp<BF16>::mma(a[1], b[1], c1);
        c2 = Lp<BF16>::mma(a[2], b[2], c2);
        c3 = Lp<BF16>::mma(a[3], b[3], c3);
        c0 = Lp<BF16>::mma(a[4], b[4], c0);
        c1 = Lp<BF16>::mma(a[5], b[5], c1);
        c2 = Lp<BF16>::mma(a[6], b[6], c2);
        c3 = Lp<BF16>::mma(a[7], b[7], c3);
    }
    const unsigned long long t1 = probe_shader_cycles(), r1 = probe_ref_ticks();
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
    sink[id] = s;
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

typedef __attribute__((address_space(3))) void probe_lds;

// Load stream: workgroup w reads region g = w % 8 + 8 * ((w / 8) / share)
// (workgroups are dealt to the 8 XCDs in turn, so `share` consecutive
// workgroups of one XCD read the same region); wavefront v's j-th load takes
// the region's 1 KB chunk (j * NW + v) mod chunks into its own ring of DEPTH+1
// LDS blocks, and waits until at most DEPTH of its loads are in flight before
// the next.  The landed data are never read.
template <int NW, int DEPTH>
__global__ __launch_bounds__(64 * NW) void load_probe_kernel(const unsigned char *__restrict__ src,
                                                             int64_t region_bytes, int share, int loads,
                                                             unsigned long long *__restrict__ clocks)
{
    __shared__ __attribute__((aligned(1024))) unsigned char ring[NW][DEPTH + 1][1024];
    const int lane = threadIdx.x & 63;
    const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t group = (int64_t)(blockIdx.x % 8) + 8 * (int64_t)((blockIdx.x / 8) / share);
    const unsigned char *p = src + group * region_bytes + 16 * lane;
    const int chunks = (int)(region_bytes / 1024);
    int c = v % chunks, slot = 0;
    __syncthreads();
    const unsigned long long t0 = probe_shader_cycles(), r0 = probe_ref_ticks();
    for (int j = 0; j < loads; ++j) {
        __builtin_amdgcn_global_load_lds(p + (int64_t)c * 1024, (probe_lds *)&ring[v][slot][0], 16, 0, 0);
        // s_waitcnt vmcnt(DEPTH - 1) (gfx9 encoding, expcnt and lgkmcnt not waited on)
        constexpr int N = DEPTH - 1;
        __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
        c += NW;
        if (c >= chunks)
            c -= chunks;
        slot = slot == DEPTH ? 0 : slot + 1;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const unsigned long long t1 = probe_shader_cycles(), r1 = probe_ref_ticks();
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// Every load-probe workgroup claims this much LDS, so that one runs per CU.
constexpr int kLoadProbeLds = 100 * 1024;

template <int NW, int DEPTH>
void launch_load(int workgroups, const void *src, int64_t region_bytes, int share, int loads,
                 unsigned long long *clocks, hipStream_t stream)
{
    constexpr int stat = NW * (DEPTH + 1) * 1024;
    static_assert(stat <= kLoadProbeLds, "ring within the claimed LDS");
    load_probe_kernel<NW, DEPTH><<<dim3((unsigned)workgroups), dim3(64 * NW), kLoadProbeLds - stat, stream>>>(
        static_cast<const unsigned char *>(src), region_bytes, share, loads, clocks);
}

}  // namespace

hipError_t launch_mfma_lp_probe(bool bf16, bool zero, int workgroups, int trips, float *sink,
                                unsigned long long *clocks, hipStream_t stream)
{
    if (bf16)
        mfma_lp_probe_kernel<true><<<dim3((unsigned)workgroups), dim3(256), 0, stream>>>(trips, zero, sink, clocks);
    else
        mfma_lp_probe_kernel<false><<<dim3((unsigned)workgroups), dim3(256), 0, stream>>>(trips, zero, sink, clocks);
    return hipGetLastError();
}

hipError_t launch_load_probe(int waves, int depth, int workgroups, const void *src, int64_t region_bytes, int share,
                             int loads, unsigned long long *clocks, hipStream_t stream)
{
#define SGEMM_LOAD_PROBE_CASE(W, D)                                                  \
    if (waves == W && depth == D) {                                                  \
        launch_load<W, D>(workgroups, src, region_bytes, share, loads, clocks, stream); \
        return hipGetLastError();                                                    \
    }
    SGEMM_LOAD_PROBE_CASE(4, 1)
    SGEMM_LOAD_PROBE_CASE(4, 2)
    SGEMM_LOAD_PROBE_CASE(4, 4)
    SGEMM_LOAD_PROBE_CASE(4, 8)
    SGEMM_LOAD_PROBE_CASE(8, 1)
    SGEMM_LOAD_PROBE_CASE(8, 2)
    SGEMM_LOAD_PROBE_CASE(8, 4)
    SGEMM_LOAD_PROBE_CASE(8, 8)
#undef SGEMM_LOAD_PROBE_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_mfma_probe(int workgroups, int trips, float *sink, unsigned long long *clocks, hipStream_t stream)
{
    mfma_probe_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, stream>>>(trips, sink, clocks);
    return hipGetLastError();
}

}  // namespace sgemm
