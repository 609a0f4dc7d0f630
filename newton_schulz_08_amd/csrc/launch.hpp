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
// Small-route weight update: p <- p * decay + step_lr * Y with decay = 1 - lr wd.
// gcoef: NULL, or per-segment clipping coefficients; matrix i's gradient is
// then read as gcoef[clip_seg] * g (in fp32, never rounded back).
hipError_t launch_prologue(int dt, const MatDesc* descs, const int* tile_prefix, int nmat, int total_tiles,
                           float* partials, int mode, float mu, int nesterov, float lr, float decay,
                           const float* gcoef, int grid, hipStream_t stream);

// Per-matrix sum of the prologue partials -> norm, 1/(norm+eps), squared.
hipError_t launch_norm_finalize(const MatDesc* descs, const int* tile_prefix, int nmat, const float* partials,
                                MatScale* scales, float* norms_out, hipStream_t stream);

// ns_steps == 0: U = X0 = Y / (||Y|| + eps) written to the caller.
hipError_t launch_apply_x0(int dt, const MatDesc* descs, const int* tile_prefix, int nmat, int total_tiles,
                           const MatScale* scales, int mode, float lr, float decay, int grid, hipStream_t stream);

// Gram products over a launch's segments, for Newton-Schulz step `step`.
//   square == 0: A = alpha X X^T (alpha = c^2 at step 0, else 1), X read from
//                the operand copy of that step (xs0 on even steps, xs1 on odd).
//   square == 1: B = cq A A + cl A (A symmetric, so A A = A A^T).
// Segments with ksplit > 1 only write one fp32 partial product per (tile,
// K slice); a second launch with reduce == 1 over a table of just those
// segments (one block per tile) sums the slices in order and stores.
hipError_t launch_syrk(int dt, const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales,
                       int step, int square, float cq, float cl, int reduce, hipStream_t stream);

// X <- g (cx X + cax M X) with M = A (poly == 0) or B (poly == 1); g = c at
// step 0, else 1.  The product reads the operand copy of step `step` and the
// epilogue writes the next step's copy (and, for bf16, the low half of the
// iterate in place).  On the last step the result U is written to the caller:
// p <- p * decay + step_lr * U (mode muon) or out = U (ns only).
hipError_t launch_ns_gemm(int dt, const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales,
                          int step, int last, int mode, float lr, float decay, float cx, float cax, int poly,
                          hipStream_t stream);

// The same two products for fp32 matrices with m' <= 2 kTile, on 128 x 128
// tiles (segments' tile grids and partial products in those tiles).
hipError_t launch_small_syrk(const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales, int step,
                             int square, float cq, float cl, int reduce, hipStream_t stream);
hipError_t launch_small_gemm(const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales, int step,
                             int last, int mode, float lr, float decay, float cx, float cax, int poly,
                             hipStream_t stream);

}  // namespace dmuon
