// Launch helper of the matrix-core probe (k_probe.hip), a measurement aid
// beside the GEMM: chains of FP32 MFMAs on register operands, timed in shader
// cycles and 100 MHz ticks per workgroup.
#pragma once
#include <hip/hip_runtime.h>

namespace sgemm {

hipError_t launch_mfma_probe(int workgroups, int trips, float *sink, unsigned long long *clocks, hipStream_t stream);

}  // namespace sgemm
