// Internal declarations of the out-of-place transpose kernels.
#pragma once

#include "sgemm_internal.h"

namespace sgemm {

// dst (cols x rows, ld_dst) <- src (rows x cols, ld_src)^T, both row-major.
struct TransposeArgs {
    const float *src;
    float *dst;
    int64_t ld_src, ld_dst;
    int rows, cols;
};

// Transpose kernel identifiers (a range of their own next to KernelId).
enum TransposeKernelId : int {
    KID_TRANSPOSE_NAIVE = 50,      // one work-item per element, contiguous reads
    KID_TRANSPOSE_LDS_PAD = 51,    // tiles through LDS with a padding column
    KID_TRANSPOSE_LDS_NOPAD = 52,  // the same tiles without it
    KID_TRANSPOSE_NARROW = 53,     // one work-item per element, contiguous writes
};

// Launch shape of the tile kernels: 64 x 64 tiles (fewer 128 x 128 tiles than
// CUs), persistent and pipelined (up to 2048 tiles) or one tile per workgroup.
enum TransposeShape : int { TSHAPE_SMALL = 0, TSHAPE_PIPE = 1, TSHAPE_STREAM = 2 };
int transpose_shape(int64_t rows, int64_t cols);

// Work units (tiles or element blocks) a kernel covers for a rows x cols
// source, and the workgroups it launches (workgroups loop over work units; the
// grid is capped).
int64_t transpose_tiles(int kid, int64_t rows, int64_t cols);
int64_t transpose_blocks(int kid, int64_t rows, int64_t cols);

// Enqueue one transpose kernel on `stream`, return hipGetLastError().  `vec`:
// src and ld_src allow 16-byte loads.
hipError_t launch_transpose(const TransposeArgs &a, int kid, bool vec, hipStream_t stream);

}  // namespace sgemm
