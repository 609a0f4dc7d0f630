// Shared definitions for the fused multi-tensor AdamW step (host planner and kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dmuon {

constexpr int kAdamChunk = 4;                                   // consecutive elements per lane and load
constexpr int kAdamChunks = 4;                                  // chunks per lane and tile
constexpr int kAdamThreads = 256;
constexpr int kAdamTile = kAdamThreads * kAdamChunk * kAdamChunks;  // 4096 elements

// One parameter tensor; lives in the workspace.
struct alignas(16) AdamDesc {
  void* p;          // device, numel contiguous elements of the parameter dtype
  const void* g;    // device, same dtype and size as p
  float* m;         // device, numel floats (first moment)
  float* v;         // device, numel floats (second moment)
  int64_t numel;
  int vec_ok;       // 1 when p and g hold whole aligned chunks and m, v are 16-byte aligned
  int pad_;
};
static_assert(sizeof(AdamDesc) == 48, "AdamDesc layout");

// Per-call constants, formed on the host from the step counter and hyper-parameters.
struct AdamArgs {
  float decay;         // 1 - lr * weight_decay
  float beta1, one_minus_beta1;
  float beta2, one_minus_beta2;
  float step_size;     // lr / (1 - beta1^t)
  float inv_bc2_sqrt;  // 1 / sqrt(1 - beta2^t)
  float eps;
};

hipError_t launch_adamw(int dt, const AdamDesc* descs, const int* tile_prefix, int n, int total_tiles,
                        const AdamArgs& args, int grid, hipStream_t stream);

}  // namespace dmuon
