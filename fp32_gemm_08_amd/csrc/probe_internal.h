// Launch helpers of the probes (k_probe.hip), measurement aids beside the
// GEMM: chains of FP32 or 16-bit MFMAs on register operands, and a stream of
// direct global->LDS loads, each timed in shader cycles and 100 MHz ticks per
// workgroup.
#pragma once
#include <hip/hip_runtime.h>

namespace sgemm {

hipError_t launch_mfma_probe(int workgroups, int trips, float *sink, unsigned long long *clocks, hipStream_t stream);
hipError_t launch_mfma_lp_probe(bool bf16, bool zero, int workgroups, int trips, float *sink,
                                unsigned long long *clocks, hipStream_t stream);
// waves in {4, 8}, depth in {1, 2, 4, 8}; anything else: hipErrorInvalidValue.
hipError_t launch_load_probe(int waves, int depth, int workgroups, const void *src, int64_t region_bytes, int share,
                             int loads, unsigned long long *clocks, hipStream_t stream);

}  // namespace sgemm
