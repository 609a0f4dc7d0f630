// Fused multi-tensor AdamW step on gfx950 (HBM-bound).
//
// The training guide ("第 4 步：创建优化器") sends every parameter that Muon
// does not take (embeddings, the output head, norm weights, biases) to a
// standard AdamW group with its own lr, betas, eps and weight decay.  The blog
// post's section "为什么需要矩阵感知优化器" gives that update as
// W <- W - alpha m_hat / (sqrt(v_hat) + eps) with bias-corrected moments.  Per
// element, in fp32, PyTorch's AdamW order:
//
//   p <- p (1 - lr wd)
//   m <- beta1 m + (1 - beta1) g
//   v <- beta2 v + (1 - beta2) g^2
//   p <- p - step_size m / (sqrt(v) / sqrt(1 - beta2^t) + eps),   step_size = lr / (1 - beta1^t)
//
// One launch covers every tensor: tensors are cut into 4096-element tiles, one
// block per tile (blocks stride over the list only past 2^22 tiles), so the
// dispatcher keeps every CU full to the end.  Each lane handles four consecutive
// elements per load, so one wave instruction covers 256 consecutive elements
// of every array (512 B of bf16, 1 KB of fp32): every access is fully
// coalesced.  All loads of a tile are issued before any arithmetic.  Bytes per
// element: bf16 parameters 12 read + 10 written, fp32 parameters 16 + 12.
#include <hip/hip_runtime.h>

#include "adamw.hpp"

namespace dmuon {
namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

template <int DT> struct AdamElem;
template <> struct AdamElem<kBF16> { using T = __bf16; using V = bf16x4_t; };
template <> struct AdamElem<kF32> { using T = float; using V = f32v4; };

__device__ __forceinline__ int find_tensor(const int* __restrict__ prefix, int n, int t) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ void adamw_elem(float& p, float g, float& m, float& v, const AdamArgs& a) {
  p *= a.decay;
  m = fmaf(a.beta1, m, a.one_minus_beta1 * g);
  v = fmaf(a.beta2, v, (a.one_minus_beta2 * g) * g);
  const float denom = fmaf(sqrtf(v), a.inv_bc2_sqrt, a.eps);
  p = fmaf(-a.step_size, m / denom, p);
}

template <int DT>
__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(const AdamDesc* __restrict__ descs,
                                                            const int* __restrict__ prefix, int n, int total_tiles,
                                                            AdamArgs a) {
  using T = typename AdamElem<DT>::T;
  using V = typename AdamElem<DT>::V;
  for (int t = blockIdx.x; t < total_tiles; t += gridDim.x) {
    const int i = find_tensor(prefix, n, t);
    const AdamDesc& d = descs[i];
    const int64_t base = static_cast<int64_t>(t - prefix[i]) * kAdamTile;
    T* pp = static_cast<T*>(d.p);
    const T* gp = static_cast<const T*>(d.g);
    if (d.vec_ok && base + kAdamTile <= d.numel) {
      V rp[kAdamChunks], rg[kAdamChunks];
      f32v4 rm[kAdamChunks], rv[kAdamChunks];
#pragma unroll
      for (int c = 0; c < kAdamChunks; ++c) {
        const int64_t e = base + (c * kAdamThreads + threadIdx.x) * kAdamChunk;
        rp[c] = *reinterpret_cast<gptr<const V>>(gmem(pp + e));
        rg[c] = *reinterpret_cast<gptr<const V>>(gmem(gp + e));
        rm[c] = *reinterpret_cast<gptr<const f32v4>>(gmem(d.m + e));
        rv[c] = *reinterpret_cast<gptr<const f32v4>>(gmem(d.v + e));
      }
      // keep every load of the tile ahead of the arithmetic
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < kAdamChunks; ++c) {
        const int64_t e = base + (c * kAdamThreads + threadIdx.x) * kAdamChunk;
        V op;
        f32v4 om, ov;
#pragma unroll
        for (int k = 0; k < kAdamChunk; ++k) {
          float p = static_cast<float>(rp[c][k]), m = rm[c][k], v = rv[c][k];
          adamw_elem(p, static_cast<float>(rg[c][k]), m, v, a);
          op[k] = static_cast<T>(p);
          om[k] = m;
          ov[k] = v;
        }
        *reinterpret_cast<gptr<V>>(gmem(pp + e)) = op;
        *reinterpret_cast<gptr<f32v4>>(gmem(d.m + e)) = om;
        *reinterpret_cast<gptr<f32v4>>(gmem(d.v + e)) = ov;
      }
    } else {
      // a tensor's last (partial) tile, or a tensor without aligned chunks
      for (int c = 0; c < kAdamChunks; ++c) {
        const int64_t e0 = base + (static_cast<int64_t>(c) * kAdamThreads + threadIdx.x) * kAdamChunk;
        for (int k = 0; k < kAdamChunk; ++k) {
          const int64_t e = e0 + k;
          if (e >= d.numel) break;
          float p = static_cast<float>(gmem(pp)[e]), m = gmem(d.m)[e], v = gmem(d.v)[e];
          adamw_elem(p, static_cast<float>(gmem(gp)[e]), m, v, a);
          gmem(pp)[e] = static_cast<T>(p);
          gmem(d.m)[e] = m;
          gmem(d.v)[e] = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_adamw(int dt, const AdamDesc* descs, const int* tile_prefix, int n, int total_tiles,
                        const AdamArgs& args, int grid, hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(adamw_kernel<kBF16>, dim3(grid), dim3(kAdamThreads), 0, stream, descs, tile_prefix, n,
                       total_tiles, args);
  else
    hipLaunchKernelGGL(adamw_kernel<kF32>, dim3(grid), dim3(kAdamThreads), 0, stream, descs, tile_prefix, n,
                       total_tiles, args);
  return hipGetLastError();
}

}  // namespace dmuon
