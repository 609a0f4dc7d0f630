// Shared definitions for per-segment gradient clipping (host planner and kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dmuon {

constexpr int kClipTile = 16384;    // elements per partial-sum tile: 8 (bf16) or 16 (fp32) 16-byte loads per thread
constexpr int kClipThreads = 256;
constexpr float kClipEps = 1e-6f;   // the +1e-6 of the clipping rule

enum ClipKind : int { kClipP2 = 0, kClipP1 = 1, kClipPInf = 2, kClipPGeneral = 3 };

// One gradient tensor; lives in the workspace.
struct alignas(16) ClipDesc {
  void* g;          // device, numel contiguous elements
  int64_t numel;
  int segment;      // index into max_norm / coefficients
  int vec_ok;       // 1 when g is 16-byte aligned (vector loads and stores)
};
static_assert(sizeof(ClipDesc) == 32, "ClipDesc layout");

// partials (one per tile) -> per-segment totals and coefficients -> in-place
// scale (scale != 0; otherwise the coefficients are left for a consumer that
// applies them on load, as the Muon step's prologue does).
hipError_t launch_clip(int dt, const ClipDesc* descs, const int* tile_prefix, int n, int total_tiles,
                       const int* seg_tile0, int nseg, const float* max_norm, int kind, float p, float* partials,
                       float* coefs, float* totals_out, int scale, int grid, hipStream_t stream);

}  // namespace dmuon
