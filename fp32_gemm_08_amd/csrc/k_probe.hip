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
#include "probe_internal.h"

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

}  // namespace

hipError_t launch_mfma_probe(int workgroups, int trips, float *sink, unsigned long long *clocks, hipStream_t stream)
{
    mfma_probe_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, stream>>>(trips, sink, clocks);
    return hipGetLastError();
}

}  // namespace sgemm
