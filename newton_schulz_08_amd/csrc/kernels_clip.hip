// Per-segment global p-norm gradient clipping on gfx950 (HBM-bound).
//
// Training guide, "梯度裁剪": the Muon-only clip is global p-norm clipping
// applied before momentum and Newton-Schulz, and the fused bucketed form
// computes every segment's norm, clip coefficient and in-place scaling while
// keeping per-segment semantics.  The rule is that of the PyTorch
// clip_grad_norm_ the guide names for the other parameters:
//
//   total_s = (sum over the segment's tensors of sum |g|^p)^(1/p)   (max |g| for p = inf)
//   coef_s  = min(max_norm_s / (total_s + 1e-6), 1)
//   g      <- coef_s * g
//
// Three launches: clip_partials_kernel reads every gradient once and writes
// one partial per 16384-element tile; clip_finalize_kernel reduces each
// segment's tiles in a fixed order (tensors are ordered by segment, so a
// segment's tiles are contiguous); clip_scale_kernel rewrites only tiles whose
// coefficient is below 1, so an unclipped step costs one read pass.
#include <hip/hip_runtime.h>

#include "clip.hpp"

namespace dmuon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <int DT> struct ClipElem;
template <> struct ClipElem<kBF16> { using T = __bf16; static constexpr int kVec = 8; };
template <> struct ClipElem<kF32> { using T = float; static constexpr int kVec = 4; };

__device__ __forceinline__ int find_tensor(const int* __restrict__ prefix, int n, int t) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// |x|^p accumulated into acc (sum), or max for p = inf.
template <int KIND>
__device__ __forceinline__ float accum(float acc, float x, float p) {
  const float a = fabsf(x);
  if constexpr (KIND == kClipP2) return fmaf(a, a, acc);
  else if constexpr (KIND == kClipP1) return acc + a;
  else if constexpr (KIND == kClipPInf) return fmaxf(acc, a);
  else return acc + powf(a, p);
}

__device__ __forceinline__ float combine(float a, float b, int kind) { return kind == kClipPInf ? fmaxf(a, b) : a + b; }

__device__ __forceinline__ float wave_reduce(float v, int kind) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = combine(v, __shfl_xor(v, o, 64), kind);
  return v;
}

// Fixed-order block reduction of one value per thread.
__device__ __forceinline__ float block_reduce(float v, int kind, float* red) {
  v = wave_reduce(v, kind);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kClipThreads / 64; ++w) r = combine(r, red[w], kind);
  __syncthreads();
  return r;
}

template <typename T> struct RawVec;
template <> struct RawVec<float> { using V = f32v4; };
template <> struct RawVec<__bf16> { using V = bf16x8_t; };

template <typename T>
__device__ __forceinline__ typename RawVec<T>::V load_raw(const T* p) {
  return *reinterpret_cast<gptr<const typename RawVec<T>::V>>(gmem(p));
}

template <typename T>
__device__ __forceinline__ void load_vec(const T* p, float* v);
template <>
__device__ __forceinline__ void load_vec<float>(const float* p, float* v) {
  const f32v4 x = *reinterpret_cast<gptr<const f32v4>>(gmem(p));
  v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
}
template <>
__device__ __forceinline__ void load_vec<__bf16>(const __bf16* p, float* v) {
  const bf16x8_t x = *reinterpret_cast<gptr<const bf16x8_t>>(gmem(p));
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(x[e]);
}
template <typename T>
__device__ __forceinline__ void store_vec(T* p, const float* v);
template <>
__device__ __forceinline__ void store_vec<float>(float* p, const float* v) {
  *reinterpret_cast<gptr<f32v4>>(gmem(p)) = f32v4{v[0], v[1], v[2], v[3]};
}
template <>
__device__ __forceinline__ void store_vec<__bf16>(__bf16* p, const float* v) {
  bf16x8_t x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<__bf16>(v[e]);
  *reinterpret_cast<gptr<bf16x8_t>>(gmem(p)) = x;
}

template <int DT, int KIND>
__global__ __launch_bounds__(kClipThreads) void clip_partials_kernel(const ClipDesc* __restrict__ descs,
                                                                     const int* __restrict__ prefix, int n,
                                                                     int total_tiles, float* __restrict__ partials,
                                                                     float p) {
  using T = typename ClipElem<DT>::T;
  constexpr int V = ClipElem<DT>::kVec;
  constexpr int kIters = kClipTile / (kClipThreads * V);
  __shared__ float red[kClipThreads / 64];
  for (int t = blockIdx.x; t < total_tiles; t += gridDim.x) {
    const int i = find_tensor(prefix, n, t);
    const ClipDesc& d = descs[i];
    const int64_t base = static_cast<int64_t>(t - prefix[i]) * kClipTile;
    const T* g = static_cast<const T*>(d.g);
    float acc = 0.0f;
    if (d.vec_ok && base + kClipTile <= d.numel) {
      // whole tile: every load in flight before any arithmetic; wave
      // instruction k covers 64 consecutive vectors (one contiguous KB)
      typename RawVec<T>::V raw[kIters];
#pragma unroll
      for (int k = 0; k < kIters; ++k) raw[k] = load_raw<T>(g + base + (k * kClipThreads + threadIdx.x) * V);
#pragma unroll
      for (int k = 0; k < kIters; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e) acc = accum<KIND>(acc, static_cast<float>(raw[k][e]), p);
    } else {
      // a tensor's last (partial) tile, or an unaligned tensor
      for (int k = 0; k < kIters; ++k) {
        const int64_t e0 = base + (static_cast<int64_t>(k) * kClipThreads + threadIdx.x) * V;
        for (int e = 0; e < V; ++e)
          if (e0 + e < d.numel) acc = accum<KIND>(acc, static_cast<float>(gmem(g)[e0 + e]), p);
      }
    }
    const float r = block_reduce(acc, KIND, red);
    if (threadIdx.x == 0) partials[t] = r;
  }
}

__global__ __launch_bounds__(kClipThreads) void clip_finalize_kernel(const int* __restrict__ seg_tile0,
                                                                     const float* __restrict__ partials,
                                                                     const float* __restrict__ max_norm, int kind,
                                                                     float p, float* __restrict__ coefs,
                                                                     float* __restrict__ totals_out) {
  __shared__ float red[kClipThreads / 64];
  const int s = blockIdx.x;
  const int t0 = seg_tile0[s], t1 = seg_tile0[s + 1];
  float acc = 0.0f;
  for (int t = t0 + threadIdx.x; t < t1; t += kClipThreads) acc = combine(acc, partials[t], kind);
  const float r = block_reduce(acc, kind, red);
  if (threadIdx.x == 0) {
    float total;
    if (kind == kClipP2) total = sqrtf(r);
    else if (kind == kClipP1 || kind == kClipPInf) total = r;
    else total = powf(r, 1.0f / p);
    const float c = max_norm[s] / (total + kClipEps);
    // clamp at 1; a NaN coefficient stays NaN, as in the reference rule
    coefs[s] = (c >= 1.0f) ? 1.0f : c;
    if (totals_out) totals_out[s] = total;
  }
}

template <int DT>
__global__ __launch_bounds__(kClipThreads) void clip_scale_kernel(const ClipDesc* __restrict__ descs,
                                                                  const int* __restrict__ prefix, int n,
                                                                  int total_tiles, const float* __restrict__ coefs) {
  using T = typename ClipElem<DT>::T;
  constexpr int V = ClipElem<DT>::kVec;
  constexpr int kIters = kClipTile / (kClipThreads * V);
  for (int t = blockIdx.x; t < total_tiles; t += gridDim.x) {
    const int i = find_tensor(prefix, n, t);
    const ClipDesc& d = descs[i];
    const float c = coefs[d.segment];
    if (c == 1.0f) continue;  // uniform per tile: an unclipped segment is not rewritten
    const int64_t base = static_cast<int64_t>(t - prefix[i]) * kClipTile;
    T* g = static_cast<T*>(d.g);
    if (d.vec_ok && base + kClipTile <= d.numel) {
      typename RawVec<T>::V raw[kIters];
#pragma unroll
      for (int k = 0; k < kIters; ++k) raw[k] = load_raw<T>(g + base + (k * kClipThreads + threadIdx.x) * V);
#pragma unroll
      for (int k = 0; k < kIters; ++k) {
        float v[V];
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = static_cast<float>(raw[k][e]) * c;
        store_vec<T>(g + base + (k * kClipThreads + threadIdx.x) * V, v);
      }
    } else {
      for (int k = 0; k < kIters; ++k) {
        const int64_t e0 = base + (static_cast<int64_t>(k) * kClipThreads + threadIdx.x) * V;
        for (int e = 0; e < V; ++e)
          if (e0 + e < d.numel) gmem(g)[e0 + e] = static_cast<T>(static_cast<float>(gmem(g)[e0 + e]) * c);
      }
    }
  }
}

}  // namespace

hipError_t launch_clip(int dt, const ClipDesc* descs, const int* tile_prefix, int n, int total_tiles,
                       const int* seg_tile0, int nseg, const float* max_norm, int kind, float p, float* partials,
                       float* coefs, float* totals_out, int scale, int grid, hipStream_t stream) {
  if (total_tiles > 0) {
    auto partials_launch = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(grid), dim3(kClipThreads), 0, stream, descs, tile_prefix, n, total_tiles,
                         partials, p);
    };
    if (dt == kBF16) {
      switch (kind) {
        case kClipP2: partials_launch(clip_partials_kernel<kBF16, kClipP2>); break;
        case kClipP1: partials_launch(clip_partials_kernel<kBF16, kClipP1>); break;
        case kClipPInf: partials_launch(clip_partials_kernel<kBF16, kClipPInf>); break;
        default: partials_launch(clip_partials_kernel<kBF16, kClipPGeneral>); break;
      }
    } else {
      switch (kind) {
        case kClipP2: partials_launch(clip_partials_kernel<kF32, kClipP2>); break;
        case kClipP1: partials_launch(clip_partials_kernel<kF32, kClipP1>); break;
        case kClipPInf: partials_launch(clip_partials_kernel<kF32, kClipPInf>); break;
        default: partials_launch(clip_partials_kernel<kF32, kClipPGeneral>); break;
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(clip_finalize_kernel, dim3(nseg), dim3(kClipThreads), 0, stream, seg_tile0, partials, max_norm,
                     kind, p, coefs, totals_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || total_tiles == 0 || !scale) return e;
  if (dt == kBF16)
    hipLaunchKernelGGL(clip_scale_kernel<kBF16>, dim3(grid), dim3(kClipThreads), 0, stream, descs, tile_prefix, n,
                       total_tiles, coefs);
  else
    hipLaunchKernelGGL(clip_scale_kernel<kF32>, dim3(grid), dim3(kClipThreads), 0, stream, descs, tile_prefix, n,
                       total_tiles, coefs);
  return hipGetLastError();
}

}  // namespace dmuon
