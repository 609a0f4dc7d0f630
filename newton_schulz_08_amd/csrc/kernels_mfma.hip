// MFMA contraction kernels for one Newton-Schulz step on gfx950.
//
// One step of the cubic map (DMuon blog post, "Muon 核心：Newton-Schulz 迭代":
// G <- 1.5 G - 0.5 G G^T G, evaluated as two products, "代码实现") is two
// launches over every matrix of the batch:
//
//   syrk_kernel    A = alpha * X X^T      lower-triangle 256x256 tiles only; each
//                                         off-diagonal tile is also stored
//                                         transposed into the upper triangle.
//   ns_gemm_kernel X <- g * (1.5 X - 0.5 A X)   fused epilogue; on the last step
//                                         it writes the update into the caller's
//                                         parameters (p -= lr * s * X) or output.
//
// Both are the same "NT" block product C[i,j] = sum_k P[i,k] Q[j,k] with both
// operands K-contiguous: the Gram uses P = Q = X (rows of X), the update uses
// P = A and Q = X^T (rows of the transposed iterate, which the previous
// epilogue keeps up to date).  Each 256-thread workgroup computes a 256x256
// tile; its four waves own 128x128 quadrants as 4x4 blocks of
// v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2_f32 (fp32).  K advances
// 128 bytes per stage (64 bf16 / 32 fp32) through a double-buffered,
// XOR-swizzled LDS tile (2 x 64 KB) that global_load_lds fills directly (no
// register staging) while the current stage is multiplied.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"

namespace dmuon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kStageBytes = 65536;   // P (32 KB) + Q (32 KB)
constexpr int kOperandBytes = 32768; // 256 rows x 128 bytes

template <int DT> struct Elem;
template <> struct Elem<kBF16> { using T = __bf16; static constexpr int kBytes = 2; };
template <> struct Elem<kF32> { using T = float; static constexpr int kBytes = 4; };

__device__ __forceinline__ float to_f32(__bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return static_cast<T>(v); }

// Map a workgroup id to a logical tile so that each XCD (workgroups are
// dispatched round-robin over the 8 XCDs) walks one contiguous range of the
// logical order, keeping operands that neighbouring tiles share in its own L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = b % 8, slot = b / 8;
  return (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
}

struct TileRef {
  int mat;   // NS descriptor index
  int bi;    // tile row
  int bj;    // tile col
  int kdim;
};

__device__ __forceinline__ TileRef locate(const SegTable& st, int logical, bool lower) {
  int si = 0;
  while (si + 1 < st.nseg && st.seg[si + 1].tile0 <= logical) ++si;
  const Segment& sg = st.seg[si];
  const int local = logical - sg.tile0;
  TileRef r;
  r.mat = sg.mat0 + local / sg.tiles_per_mat;
  const int t = local % sg.tiles_per_mat;
  r.kdim = sg.kdim;
  if (lower) {
    // t -> (bi, bj), bj <= bi, row-major over the lower triangle
    int bi = static_cast<int>((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
    while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
    while (bi * (bi + 1) / 2 > t) --bi;
    r.bi = bi;
    r.bj = t - bi * (bi + 1) / 2;
  } else {
    // groups of kGroupRows tile rows, walked column by column, so the tiles
    // resident at one time share few A row panels and X^T row panels
    constexpr int kGroupRows = 4;
    const int gsz = kGroupRows * sg.tn;
    const int grp = t / gsz;
    const int first = grp * kGroupRows;
    const int gh = min(sg.tm - first, kGroupRows);
    const int within = t - grp * gsz;
    r.bi = first + within % gh;
    r.bj = within / gh;
  }
  return r;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) const void* gbl_ptr_t;

// Accumulate the 256x256 tile of P * Q^T into acc.  P0/Q0 point at the first
// row of each 256-row panel; ld*_bytes are row pitches; kbytes the contraction
// length in bytes (a multiple of 128).
//
// Global -> LDS: global_load_lds_dwordx4 writes lane l's 16 bytes to
// LDS[M0 + 16 l], so one wave instruction fills 8 rows x 128 bytes.  Lane l
// fetches chunk (l & 7) ^ (row & 7) of its row, which stores the tile in the
// XOR-swizzled layout the fragment reads expect, with no VGPR staging.  Each
// wave loads rows [64 w, 64 w + 64) of both operands (8 + 8 instructions per
// stage).
template <int DT>
__device__ __forceinline__ void block_product(const char* __restrict__ P0, long ldp_bytes,
                                              const char* __restrict__ Q0, long ldq_bytes,
                                              int kbytes, char* lds, f32x16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int li = lane & 31, lh = lane >> 5;

  const int lrow = lane >> 3;                    // row within an 8-row group
  const int lchunk = (lane & 7) ^ lrow;          // source chunk for the swizzled slot
  const char* gp = P0 + static_cast<long>(wave * 64 + lrow) * ldp_bytes + lchunk * 16;
  const char* gq = Q0 + static_cast<long>(wave * 64 + lrow) * ldq_bytes + lchunk * 16;
  const long grp_p = 8L * ldp_bytes, grp_q = 8L * ldq_bytes;
  char* lds_wave = lds + wave * 64 * 128;

  auto issue = [&](int stage, int kb) {
    char* dp = lds_wave + stage * kStageBytes;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(gp + u * grp_p + kb), (lds_ptr_t)(dp + u * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(gq + u * grp_q + kb), (lds_ptr_t)(dp + kOperandBytes + u * 1024),
                                       16, 0, 0);
    }
  };

  // fragment reads: row (block * 32 + li), chunk (2 s + lh) ^ (li & 7)
  const int frag_row = li * 128;
  const int sw = li & 7;

  const int nk = kbytes / 128;
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    // branch-free body: the last iteration re-loads the final stage into the
    // idle buffer (in bounds, never read) so the loop stays one basic block
    const int next_kb = min(kt + 1, nk - 1) * 128;
    const char* sp = lds + (kt & 1) * kStageBytes + wr * 128 * 128 + frag_row;
    const char* sq = lds + (kt & 1) * kStageBytes + kOperandBytes + wc * 128 * 128 + frag_row;
    if constexpr (DT == kBF16) {
      // fragments of sub-step s + 1 are read while sub-step s multiplies
      bf16x8 a[2][4], b[2][4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        a[0][x] = *reinterpret_cast<const bf16x8*>(sp + x * 32 * 128 + ((lh ^ sw) << 4));
        b[0][x] = *reinterpret_cast<const bf16x8*>(sq + x * 32 * 128 + ((lh ^ sw) << 4));
      }
      issue((kt + 1) & 1, next_kb);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int cur = s & 1;
        if (s + 1 < 4) {
          const int co = (((2 * (s + 1) + lh) ^ sw) << 4);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            a[cur ^ 1][x] = *reinterpret_cast<const bf16x8*>(sp + x * 32 * 128 + co);
            b[cur ^ 1][x] = *reinterpret_cast<const bf16x8*>(sq + x * 32 * 128 + co);
          }
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][mi], b[cur][ni], acc[mi][ni], 0, 0, 0);
      }
    } else {
      issue((kt + 1) & 1, next_kb);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int co = (((2 * s + lh) ^ sw) << 4);
        f32x4 a[4], b[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          a[x] = *reinterpret_cast<const f32x4*>(sp + x * 32 * 128 + co);
          b[x] = *reinterpret_cast<const f32x4*>(sq + x * 32 * 128 + co);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mi][e], b[ni][e], acc[mi][ni], 0, 0, 0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads, 1) void syrk_kernel(const MatDesc* __restrict__ descs, SegTable st,
                                                          const MatScale* __restrict__ scales, int first_step) {
  using T = typename Elem<DT>::T;
  constexpr int EB = Elem<DT>::kBytes;
  __shared__ __attribute__((aligned(16))) char lds[2 * kStageBytes];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const TileRef tr = locate(st, logical, true);
  const MatDesc& d = descs[tr.mat];
  const int mp = d.mp, np = d.np;
  const char* xs = static_cast<const char*>(d.xs);
  const long ld = static_cast<long>(np) * EB;

  f32x16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x16{};

  block_product<DT>(xs + static_cast<long>(tr.bi) * kTile * ld, ld, xs + static_cast<long>(tr.bj) * kTile * ld, ld,
                    np * EB, lds, acc);

  const float alpha = first_step ? scales[tr.mat].c2 : 1.0f;
  T* a = static_cast<T*>(d.a);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1, li = lane & 31, lh = lane >> 5;
  const int R0 = tr.bi * kTile + wr * 128, C0 = tr.bj * kTile + wc * 128;
  const bool mirror = tr.bi != tr.bj;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = C0 + ni * 32 + li;
        const int row0 = R0 + mi * 32 + 8 * g + 4 * lh;
        T v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = from_f32<T>(acc[mi][ni][4 * g + q] * alpha);
          a[static_cast<long>(row0 + q) * mp + col] = v[q];
        }
        if (mirror) {
          T* dst = a + static_cast<long>(col) * mp + row0;
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[q] = v[q];
        }
      }
}

template <int DT>
__global__ __launch_bounds__(kThreads, 1) void ns_gemm_kernel(const MatDesc* __restrict__ descs, SegTable st,
                                                             const MatScale* __restrict__ scales, int step,
                                                             int last, int mode, float lr) {
  using T = typename Elem<DT>::T;
  constexpr int EB = Elem<DT>::kBytes;
  __shared__ __attribute__((aligned(16))) char lds[2 * kStageBytes];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const TileRef tr = locate(st, logical, false);
  const MatDesc& d = descs[tr.mat];
  const int mp = d.mp, np = d.np;
  const char* a = static_cast<const char*>(d.a);
  const char* xt_in = static_cast<const char*>((step & 1) ? d.xt1 : d.xt0);
  const long lda = static_cast<long>(mp) * EB;

  f32x16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x16{};

  block_product<DT>(a + static_cast<long>(tr.bi) * kTile * lda, lda, xt_in + static_cast<long>(tr.bj) * kTile * lda,
                    lda, mp * EB, lds, acc);

  const float gamma = (step == 0) ? scales[tr.mat].c : 1.0f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1, li = lane & 31, lh = lane >> 5;
  const int R0 = tr.bi * kTile + wr * 128, C0 = tr.bj * kTile + wc * 128;
  float* xm = d.xm;

  if (!last) {
    T* xs = static_cast<T*>(d.xs);
    T* xt_out = static_cast<T*>((step & 1) ? d.xt0 : d.xt1);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = C0 + ni * 32 + li;
          const int row0 = R0 + mi * 32 + 8 * g + 4 * lh;
          T tv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const long idx = static_cast<long>(row0 + q) * np + col;
            const float xn = gamma * (1.5f * xm[idx] - 0.5f * acc[mi][ni][4 * g + q]);
            xm[idx] = xn;
            tv[q] = from_f32<T>(xn);
            if constexpr (DT == kBF16) xs[idx] = tv[q];
          }
          T* dst = xt_out + static_cast<long>(col) * mp + row0;
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[q] = tv[q];
        }
    return;
  }

  // last step: U = X_k in the caller's orientation
  const int m = d.m, n = d.n;
  const bool trn = d.tr != 0;
  T* p = static_cast<T*>(d.p);
  float* upd = d.upd;
  const float step_lr = -lr * d.lr_scale;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = C0 + ni * 32 + li;
        const int row0 = R0 + mi * 32 + 8 * g + 4 * lh;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = row0 + q;
          const float u = gamma * (1.5f * xm[static_cast<long>(row) * np + col] - 0.5f * acc[mi][ni][4 * g + q]);
          // wide (row, col) is caller (row, col), or caller (col, row) when transposed
          const int orow = trn ? col : row, ocol = trn ? row : col;
          if (orow < m && ocol < n) {
            const long o = static_cast<long>(orow) * n + ocol;
            if (mode == kModeMuon) {
              p[o] = from_f32<T>(fmaf(step_lr, u, to_f32(p[o])));
              if (upd) upd[o] = u;
            } else {
              p[o] = from_f32<T>(u);
            }
          }
        }
      }
}

}  // namespace

hipError_t launch_syrk(int dt, const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales,
                       int first_step, hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(syrk_kernel<kBF16>, dim3(ntiles), dim3(kThreads), 0, stream, descs, st, scales, first_step);
  else
    hipLaunchKernelGGL(syrk_kernel<kF32>, dim3(ntiles), dim3(kThreads), 0, stream, descs, st, scales, first_step);
  return hipGetLastError();
}

hipError_t launch_ns_gemm(int dt, const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales,
                          int step, int last, int mode, float lr, hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(ns_gemm_kernel<kBF16>, dim3(ntiles), dim3(kThreads), 0, stream, descs, st, scales, step, last,
                       mode, lr);
  else
    hipLaunchKernelGGL(ns_gemm_kernel<kF32>, dim3(ntiles), dim3(kThreads), 0, stream, descs, st, scales, step, last,
                       mode, lr);
  return hipGetLastError();
}

}  // namespace dmuon
