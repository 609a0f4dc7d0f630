// HBM-bound kernels of the Muon step on gfx950.
//
// prologue_kernel  -- one pass over every matrix, 256 threads per tile (16 x 256
//   tiles; 64 x 64 for tall Newton-Schulz matrices):
//     buf <- mu * buf + g                       (blog post VanillaMuon: mul_ then add_)
//     Y   <- g + mu * buf  or  buf              (training guide: nesterov ns_input)
//     partial sums of Y^2 per 16 x 64 block     (Frobenius norm of the NS input)
//   small matrices (numel < 100000, training guide "编写 Predicate"):
//     p <- p (1 - lr wd) - lr * s * Y, update_out <- Y  (blog VanillaMuon non-matrix
//     branch, with the decoupled weight decay of the training guide's optimizer)
//   Newton-Schulz matrices: Y is written, unnormalised, in the wide
//   orientation as the iterate (fp32, or for bf16 the pair hi = bf16(Y),
//   lo = bf16(Y - hi)); a tall matrix's tile goes through an LDS transpose so
//   both sides stay coalesced.
//   The 1/||Y|| scale is folded into the first Newton-Schulz step instead of a
//   second pass.
// norm_finalize_kernel -- fixed-order sum of each matrix's block partials.
//
// The sum of squares is reduced in one canonical order over the wide
// orientation, whatever tile shape produced the values: the wide iterate
// (Mp x Np) is cut into 16-row x 64-column blocks; a block's partial is the sum
// over its 16 rows (fixed pairwise tree) of row sums, each row sum a 16-lane
// butterfly over four-element quads, each quad an fmaf chain in column order.
// Block partials are stored row-major over the block grid.  A matrix and its
// transpose therefore get bitwise the same norm, and since their iterates are
// the same wide matrix, bitwise the same Newton-Schulz result.
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

// Sum over the 16 lanes of an aligned lane group (every lane gets the same
// value: each butterfly level adds the same two operands in either order).
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum of squares of a four-element quad, in column order.
__device__ __forceinline__ float quad_ss(const float (&y)[4]) {
  float q = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) q = fmaf(y[e], y[e], q);
  return q;
}

// A block's 16 row sums, added in a fixed pairwise tree.
__device__ __forceinline__ float block_sum(const float* r) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = r[2 * i] + r[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = a[2 * i] + a[2 * i + 1];
  return (a[0] + a[1]) + (a[2] + a[3]);
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
                                                              float decay, const float* __restrict__ gcoef) {
  using T = typename Elem<DT>::T;
  __shared__ float tile[kEwTile][kEwTile + 1];
  __shared__ float rowsum[4][16];   // row sums of the tile's four 16 x 64 blocks
  const int tid = threadIdx.x;
  const int quad = tid & 15;        // four-element quad within a block row

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
        if (gcoef) {
          // clipped gradient (training guide, "梯度裁剪": clipping precedes momentum)
          const float cf = gcoef[d.clip_seg];
#pragma unroll
          for (int e = 0; e < 4; ++e) g[pass][e] *= cf;
        }
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
      if (ns && trn) {
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[rl][cl + e] = y[e];
      } else {
        // 16 x 256 tile in the wide orientation: block (tid >> 4) & 3, block row rl
        const float rs = row16_sum(quad_ss(y));
        if (quad == 0) rowsum[(tid >> 4) & 3][rl] = rs;
        // the covered extent is padded to 256, so every tile position exists;
        // wide: caller rows are rows of X
        if (ns) store_iterate<DT>(d, static_cast<long>(r) * np + c, y);
      }
    }

    long pidx;   // the tile's first block partial; its blocks follow at stride bstride
    int bstride;
    if (ns && trn) {
      // tall: caller columns are rows of X, written through the LDS tile.
      // Pass p is block p of the tile's 64 wide rows, block row rl0.
      __syncthreads();
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int j = rl0 + rstep * pass;  // input column -> output row
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = tile[cl + e][j];
        const float rs = row16_sum(quad_ss(v));
        if (quad == 0) rowsum[pass][rl0] = rs;
        store_iterate<DT>(d, static_cast<long>(c0 + j) * np + r0 + cl, v);
      }
      // wide block grid (Mp / 16) x (Np / 64): this tile is block column
      // r0 / 64 of block rows c0 / 16 .. c0 / 16 + 3
      const int bcols = d.ew_rows / kEwTile;
      pidx = static_cast<long>(c0 / 16) * bcols + r0 / kEwTile;
      bstride = bcols;
    } else {
      // wide block grid (rows / 16) x (cols / 64): block row r0 / 16, block
      // columns c0 / 64 .. c0 / 64 + 3, i.e. 4 local .. 4 local + 3
      pidx = 4L * local;
      bstride = 1;
    }
    __syncthreads();
    if (tid < 4) partials[4L * d.ew_tile0 + pidx + static_cast<long>(tid) * bstride] = block_sum(rowsum[tid]);
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
  const long t0 = 4L * prefix[i], t1 = 4L * prefix[i + 1];   // four block partials per tile
  float s = 0.0f;
  for (long t = t0 + threadIdx.x; t < t1; t += kEwThreads) s += partials[t];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float ss = (red[0] + red[1]) + (red[2] + red[3]);
    const float norm = sqrtf(ss);
    // The scale is folded into the first Newton-Schulz step: its Gram product
    // accumulates the unnormalised Y Y^T in fp32 and multiplies by c^2.  Both
    // stay in range (entries below ||Y||^2, c^2 at least the smallest normal
    // float) while ||Y|| < 2^63; beyond that (or an overflowed sum) the scale
    // is NaN, so the matrix's update is NaN as for a non-finite gradient.
    const float c = norm < kMaxFoldedNorm ? 1.0f / (norm + kNormEps) : __builtin_nanf("");
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
                           float* partials, int mode, float mu, int nesterov, float lr, float decay,
                           const float* gcoef, int grid, hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(prologue_kernel<kBF16>, dim3(grid), dim3(kEwThreads), 0, stream, descs, tile_prefix, nmat,
                       total_tiles, partials, mode, mu, nesterov, lr, decay, gcoef);
  else
    hipLaunchKernelGGL(prologue_kernel<kF32>, dim3(grid), dim3(kEwThreads), 0, stream, descs, tile_prefix, nmat,
                       total_tiles, partials, mode, mu, nesterov, lr, decay, gcoef);
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
