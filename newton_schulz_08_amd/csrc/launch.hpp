// Host-side launch wrappers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace dmuon {

constexpr int kMaxSegPerLaunch = 16;

// Segments of one contraction launch, passed by value as a kernel argument.
struct SegTable {
  int nseg;
  int pad_[3];
  Segment seg[kMaxSegPerLaunch];
};

// Fused momentum / Nesterov / norm partials / small-matrix update / iterate
// materialisation, over `total_tiles` 64x64 tiles of all matrices.
hipError_t launch_prologue(int dt, const MatDesc* descs, const int* tile_prefix, int nmat, int total_tiles,
                           float* partials, int mode, float mu, int nesterov, float lr, int grid,
                           hipStream_t stream);

// Per-matrix sum of the prologue partials -> norm, 1/(norm+eps), squared.
hipError_t launch_norm_finalize(const MatDesc* descs, const int* tile_prefix, int nmat, const float* partials,
                                MatScale* scales, float* norms_out, hipStream_t stream);

// ns_steps == 0: U = X0 = Y / (||Y|| + eps) written to the caller.
hipError_t launch_apply_x0(int dt, const MatDesc* descs, const int* tile_prefix, int nmat, int total_tiles,
                           const MatScale* scales, int mode, float lr, int grid, hipStream_t stream);

hipError_t launch_syrk(int dt, const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales,
                       int first_step, hipStream_t stream);

hipError_t launch_ns_gemm(int dt, const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales,
                          int step, int last, int mode, float lr, hipStream_t stream);

}  // namespace dmuon
