// HBM-bound kernels of the Muon step on gfx950.
//
// prologue_kernel  -- one pass over every matrix, 256 threads per tile (16 x 256
//   tiles; 64 x 64 for tall Newton-Schulz matrices):
//     buf <- mu * buf + g                       (blog post VanillaMuon: mul_ then add_)
//     Y   <- g + mu * buf  or  buf              (training guide: nesterov ns_input)
//     partial sum of Y^2 per tile               (Frobenius norm of the NS input)
//   small matrices (numel < 100000, training guide "编写 Predicate"):
//     p <- p (1 - lr wd) - lr * s * Y, update_out <- Y  (blog VanillaMuon non-matrix
//     branch, with the decoupled weight decay of the training guide's optimizer)
//   Newton-Schulz matrices: Y is written, unnormalised, in the wide
//   orientation as the iterate (fp32, or for bf16 the pair hi = bf16(Y),
//   lo = bf16(Y - hi)); a tall matrix's tile goes through an LDS transpose so
//   both sides stay coalesced.
//   The 1/||Y|| scale is folded into the first Newton-Schulz step instead of a
//   second pass.
// norm_finalize_kernel -- fixed-order sum of each matrix's tile partials.
// apply_x0_kernel -- ns_steps == 0 only: U = Y / (||Y|| + eps) to the caller.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"

namespace dmuon {
namespace {

template <int DT> struct Elem;
template <> struct Elem<kBF16> { using T = __bf16; };
template <> struct Elem<kF32> { using T = float; };

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(__bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return static_cast<T>(v); }

template <typename T>
__device__ __forceinline__ void load4(const T* __restrict__ src, bool vec, int valid, float (&v)[4]) {
  if (vec) {
    if constexpr (sizeof(T) == 2) {
      const bf16x4 x = *reinterpret_cast<gptr<const bf16x4>>(gmem(src));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = to_f32(x[e]);
    } else {
      const f32v4 x = *reinterpret_cast<gptr<const f32v4>>(gmem(src));
      v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (e < valid) ? to_f32(gmem(src)[e]) : 0.0f;
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* __restrict__ dst, bool vec, int valid, const float (&v)[4]) {
  if (vec) {
    if constexpr (sizeof(T) == 2) {
      bf16x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = from_f32<T>(v[e]);
      *reinterpret_cast<gptr<bf16x4>>(gmem(dst)) = x;
    } else {
      *reinterpret_cast<gptr<f32v4>>(gmem(dst)) = f32v4{v[0], v[1], v[2], v[3]};
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < valid) gmem(dst)[e] = from_f32<T>(v[e]);
  }
}

// Four consecutive elements of the wide iterate X at element offset w.  fp32:
// X itself (xm, the same memory as xs0).  bf16: the pair hi = bf16(X) (the
// operand copy xs0) and lo = bf16(X - hi) (xm).
template <int DT>
__device__ __forceinline__ void store_iterate(const MatDesc& d, long w, const float (&x)[4]) {
  if constexpr (DT == kBF16) {
    float hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi[e] = to_f32(from_f32<__bf16>(x[e]));
      lo[e] = x[e] - hi[e];
    }
    store4(static_cast<__bf16*>(d.xs0) + w, true, 4, hi);
    store4(static_cast<__bf16*>(d.xm) + w, true, 4, lo);
  } else {
    store4(static_cast<float*>(d.xm) + w, true, 4, x);
  }
}
template <int DT>
__device__ __forceinline__ void load_iterate(const MatDesc& d, long w, float (&x)[4]) {
  if constexpr (DT == kBF16) {
    float lo[4];
    load4(static_cast<const __bf16*>(d.xs0) + w, true, 4, x);
    load4(static_cast<const __bf16*>(d.xm) + w, true, 4, lo);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] += lo[e];
  } else {
    load4(static_cast<const float*>(d.xm) + w, true, 4, x);
  }
}

__device__ __forceinline__ int find_matrix(const int* __restrict__ prefix, int nmat, int t) {
  int lo = 0, hi = nmat - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Tile shapes (4096 elements, 256 threads, four passes of four elements per
// thread).  A tall Newton-Schulz matrix is written transposed, so its tiles
// are 64 x 64 and go through LDS; every other matrix uses 16 x 256 tiles, in
// which one wave instruction covers 256 consecutive elements of one row.
struct EwShape {
  int rows, cols, tpr;  // tile rows, tile cols, threads per row
};
__device__ __forceinline__ EwShape ew_shape(bool transposed) {
  return transposed ? EwShape{kEwTile, kEwTile, kEwTile / 4} : EwShape{kEwRowTileRows, kEwRowTileCols, kEwRowTileCols / 4};
}

template <int DT>
__global__ __launch_bounds__(kEwThreads) void prologue_kernel(const MatDesc* __restrict__ descs,
                                                              const int* __restrict__ prefix, int nmat,
                                                              int total_tiles, float* __restrict__ partials,
                                                              int mode, float mu, int nesterov, float lr,
                                                              float decay) {
  using T = typename Elem<DT>::T;
  __shared__ float tile[kEwTile][kEwTile + 1];
  __shared__ float red[kEwThreads / 64];
  const int tid = threadIdx.x;

  for (int t = blockIdx.x; t < total_tiles; t += gridDim.x) {
    const MatDesc& d = descs[find_matrix(prefix, nmat, t)];
    const int m = d.m, n = d.n;
    const bool ns = d.ns != 0, trn = d.tr != 0;
    const EwShape sh = ew_shape(ns && trn);
    const int local = t - d.ew_tile0;
    const int tr_ = local / d.ew_tiles_c;
    const int r0 = tr_ * sh.rows, c0 = (local - tr_ * d.ew_tiles_c) * sh.cols;
    const int cl = (tid % sh.tpr) * 4;   // 4 consecutive columns
    const int rl0 = tid / sh.tpr;        // rows rl0 + rstep * pass
    const int rstep = kEwThreads / sh.tpr;
    const int np = d.np;
    const float step_lr = -lr * d.lr_scale;
    float ss = 0.0f;

    // every load of the tile first, then the arithmetic and the stores
    float g[4][4], b[4][4], pv[4][4];
    bool in[4], vec[4];
    int valid[4];
    long o[4];
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int r = r0 + rl0 + rstep * pass, c = c0 + cl;
      in[pass] = r < m && c < n;
      valid[pass] = in[pass] ? min(4, n - c) : 0;
      vec[pass] = d.vec_ok && valid[pass] == 4;
      o[pass] = static_cast<long>(r) * n + c;
      if (in[pass]) {
        load4(static_cast<const T*>(d.g) + o[pass], vec[pass], valid[pass], g[pass]);
        if (mode == kModeMuon) load4(d.buf + o[pass], vec[pass], valid[pass], b[pass]);
        if (!ns) load4(static_cast<const T*>(d.p) + o[pass], vec[pass], valid[pass], pv[pass]);
      }
    }
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int rl = rl0 + rstep * pass;
      const int r = r0 + rl, c = c0 + cl;
      float y[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (in[pass]) {
        if (mode == kModeMuon) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            b[pass][e] = fmaf(mu, b[pass][e], g[pass][e]);
            y[e] = nesterov ? fmaf(mu, b[pass][e], g[pass][e]) : b[pass][e];
          }
          store4(d.buf + o[pass], vec[pass], valid[pass], b[pass]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = g[pass][e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e >= valid[pass]) y[e] = 0.0f;
        if (!ns) {
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[pass][e] = fmaf(step_lr, y[e], pv[pass][e] * decay);
          store4(static_cast<T*>(d.p) + o[pass], vec[pass], valid[pass], pv[pass]);
          if (d.upd) store4(d.upd + o[pass], vec[pass], valid[pass], y);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf(y[e], y[e], ss);
      if (ns) {
        // the covered extent is padded to 256, so every tile position exists
        if (!trn) {
          // wide: caller rows are rows of X
          store_iterate<DT>(d, static_cast<long>(r) * np + c, y);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) tile[rl][cl + e] = y[e];
        }
      }
    }

    if (ns && trn) {
      // tall: caller columns are rows of X, written through the LDS tile
      __syncthreads();
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int j = rl0 + rstep * pass;  // input column -> output row
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = tile[cl + e][j];
        store_iterate<DT>(d, static_cast<long>(c0 + j) * np + r0 + cl, v);
      }
    }

    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0) partials[t] = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
  }
}

__global__ __launch_bounds__(kEwThreads) void norm_finalize_kernel(const MatDesc* __restrict__ descs,
                                                                   const int* __restrict__ prefix,
                                                                   const float* __restrict__ partials,
                                                                   MatScale* __restrict__ scales,
                                                                   float* __restrict__ norms_out) {
  __shared__ float red[kEwThreads / 64];
  const int i = blockIdx.x;
  const int t0 = prefix[i], t1 = prefix[i + 1];
  float s = 0.0f;
  for (int t = t0 + threadIdx.x; t < t1; t += kEwThreads) s += partials[t];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float ss = (red[0] + red[1]) + (red[2] + red[3]);
    const float norm = sqrtf(ss);
    const float c = 1.0f / (norm + kNormEps);
    MatScale sc;
    sc.c = c;
    sc.c2 = c * c;
    sc.norm = norm;
    sc.pad_ = 0.0f;
    scales[i] = sc;
    if (norms_out) norms_out[descs[i].out_index] = norm;
  }
}

template <int DT>
__global__ __launch_bounds__(kEwThreads) void apply_x0_kernel(const MatDesc* __restrict__ descs,
                                                              const int* __restrict__ prefix, int nmat,
                                                              int total_tiles, const MatScale* __restrict__ scales,
                                                              int mode, float lr, float decay) {
  using T = typename Elem<DT>::T;
  __shared__ float tile[kEwTile][kEwTile + 1];
  const int tid = threadIdx.x;
  for (int t = blockIdx.x; t < total_tiles; t += gridDim.x) {
    const int mi = find_matrix(prefix, nmat, t);
    const MatDesc& d = descs[mi];
    if (!d.ns) continue;  // uniform per tile
    const EwShape sh = ew_shape(d.tr != 0);
    const int local = t - d.ew_tile0;
    const int tr_ = local / d.ew_tiles_c;
    const int r0 = tr_ * sh.rows, c0 = (local - tr_ * d.ew_tiles_c) * sh.cols;
    const int cl = (tid % sh.tpr) * 4;
    const int rl0 = tid / sh.tpr;
    const int rstep = kEwThreads / sh.tpr;
    const int m = d.m, n = d.n, np = d.np;
    const float sc = scales[mi].c;
    const float step_lr = -lr * d.lr_scale;
    if (d.tr) {
      // caller (r, c) is wide (c, r): stage the wide tile rows c0.., cols r0..
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int j = rl0 + rstep * pass;
        float v[4];
        load_iterate<DT>(d, static_cast<long>(c0 + j) * np + r0 + cl, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[j][cl + e] = v[e];
      }
      __syncthreads();
    }
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int rl = rl0 + rstep * pass;
      const int r = r0 + rl, c = c0 + cl;
      if (r < m && c < n) {
        const int valid = min(4, n - c);
        const bool vec = d.vec_ok && valid == 4;
        float u[4];
        if (d.tr) {
#pragma unroll
          for (int e = 0; e < 4; ++e) u[e] = tile[cl + e][rl];
        } else {
          load_iterate<DT>(d, static_cast<long>(r) * np + c, u);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] *= sc;
        const long o = static_cast<long>(r) * n + c;
        T* p = static_cast<T*>(d.p) + o;
        if (mode == kModeMuon) {
          float pv[4];
          load4(p, vec, valid, pv);
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] = fmaf(step_lr, u[e], pv[e] * decay);
          store4(p, vec, valid, pv);
          if (d.upd) store4(d.upd + o, vec, valid, u);
        } else {
          store4(p, vec, valid, u);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_prologue(int dt, const MatDesc* descs, const int* tile_prefix, int nmat, int total_tiles,
                           float* partials, int mode, float mu, int nesterov, float lr, float decay, int grid,
                           hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(prologue_kernel<kBF16>, dim3(grid), dim3(kEwThreads), 0, stream, descs, tile_prefix, nmat,
                       total_tiles, partials, mode, mu, nesterov, lr, decay);
  else
    hipLaunchKernelGGL(prologue_kernel<kF32>, dim3(grid), dim3(kEwThreads), 0, stream, descs, tile_prefix, nmat,
                       total_tiles, partials, mode, mu, nesterov, lr, decay);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const MatDesc* descs, const int* tile_prefix, int nmat, const float* partials,
                                MatScale* scales, float* norms_out, hipStream_t stream) {
  if (nmat <= 0) return hipSuccess;
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(nmat), dim3(kEwThreads), 0, stream, descs, tile_prefix, partials,
                     scales, norms_out);
  return hipGetLastError();
}

hipError_t launch_apply_x0(int dt, const MatDesc* descs, const int* tile_prefix, int nmat, int total_tiles,
                           const MatScale* scales, int mode, float lr, float decay, int grid, hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(apply_x0_kernel<kBF16>, dim3(grid), dim3(kEwThreads), 0, stream, descs, tile_prefix, nmat,
                       total_tiles, scales, mode, lr, decay);
  else
    hipLaunchKernelGGL(apply_x0_kernel<kF32>, dim3(grid), dim3(kEwThreads), 0, stream, descs, tile_prefix, nmat,
                       total_tiles, scales, mode, lr, decay);
  return hipGetLastError();
}

}  // namespace dmuon
