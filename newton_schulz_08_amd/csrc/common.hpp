// Shared definitions between the host planner and the gfx950 kernels.
//
// Data layout in HBM (per Newton-Schulz matrix, "wide" orientation: m' rows =
// min(rows, cols), n' cols = max(rows, cols); both padded up to multiples of
// kTile so the contraction kernels run without bounds checks):
//
//   xs0, xs1  dtype  Mp x Np  row-major  operand copies of X, one per step
//                                        parity: step k reads xs[k % 2] (Gram and
//                                        update) and its update epilogue writes
//                                        xs[(k + 1) % 2].  fp32: the iterate itself;
//                                        bf16: hi = bf16(X).
//   xm        bf16   Mp x Np  row-major  bf16 only: lo = bf16(X - hi), updated in
//                                        place (fp32: the same memory as xs0)
//   a         dtype  Mp x Mp  row-major  Gram matrix X X^T (symmetric)
//   b         dtype  Mp x Mp  row-major  c2 A A + c1 A, three-term maps only
//
// Padding rows/cols hold zeros, which every stage preserves.
#pragma once

#include <stdint.h>

namespace dmuon {

constexpr int kTile = 256;           // MFMA block tile (rows and cols)
constexpr int kSmallTile = 128;      // block tile of the fp32 kernels for m' <= 2 kTile
constexpr int kEwTile = 64;          // elementwise tile of a transposed (tall) matrix: 64 x 64
constexpr int kEwRowTileRows = 16;   // elementwise tile of every other matrix: 16 x 256
constexpr int kEwRowTileCols = 256;
constexpr int kEwThreads = 256;
constexpr float kNormEps = 1e-7f;    // blog post: G / (G.norm() + 1e-7)
// Largest ||Y||_F whose scale can be folded into the first Newton-Schulz step
// in fp32 (||Y||^2 and 1 / ||Y||^2 both normal floats).
constexpr float kMaxFoldedNorm = 9223372036854775808.0f;   // 2^63

enum Dtype : int { kF32 = 0, kBF16 = 1 };

// Prologue modes.
enum PrologueMode : int {
  kModeMuon = 0,   // momentum + Nesterov + route
  kModeNsOnly = 1, // Y = x (dmuon_ns_batched)
};

// One matrix of the call.  Lives in the workspace; 128 bytes.
struct alignas(16) MatDesc {
  const void* g;     // grad (muon step) or x_in (ns only)
  float* buf;        // momentum buffer (muon step) or nullptr
  void* p;           // params (muon step) or x_out (ns only)
  float* upd;        // optional fp32 update output (original orientation)
  void* xm;          // workspace, Mp x Np.  fp32: the iterate X (the same memory as xs0).
                     // bf16: the low half of the iterate, X - bf16(X) rounded to bf16, so
                     // that X = hi + lo with hi the operand copy (16 significant bits);
                     // updated in place.
  void* xs0;         // workspace: operand copy of X (dtype), Mp x Np, read on even steps
  void* xs1;         // workspace: operand copy of X, Mp x Np, read on odd steps (fp32: the
                     // iterate itself alternates between xs0 and xs1)
  void* a;           // workspace: Gram matrix, Mp x Mp
  void* b;           // workspace: c1 A + c2 A^2 for three-term maps, Mp x Mp (else nullptr)
  int m, n;          // caller shape (rows, cols)
  int mp, np;        // padded wide dims (NS route only)
  int tr;            // 1 when rows > cols (iterate on the transpose)
  int ns;            // 1 = Newton-Schulz route, 0 = elementwise route
  int out_index;     // position in the caller's arrays (norms_out)
  int ew_tile0;      // first prologue tile of this matrix
  int ew_tiles_c;    // prologue tiles along the covered column extent
  int ew_rows;       // covered extent (rows) for the prologue
  int ew_cols;       // covered extent (cols) for the prologue
  int vec_ok;        // 1 when 4-element vector access is aligned for g/buf/p/upd
  float lr_scale;
  int clip_seg;      // clipping segment of the gradient (its coefficient scales g on load)
};
static_assert(sizeof(MatDesc) == 128, "MatDesc layout");

// A run of equally shaped Newton-Schulz matrices inside one contraction launch.
struct alignas(16) Segment {
  int tile0;          // first logical tile of the segment
  int ntiles;         // count * tiles_per_mat
  int tiles_per_mat;
  int mat0;           // first entry in the NS descriptor list
  int tm, tn;         // tile grid: rows, cols of the launch's tiles (kTile, or kSmallTile for the
                      // small fp32 kernels; SYRK: tm == tn)
  int kdim;           // contraction length in elements
  int full;           // Gram only: 1 = every tile, no mirror (measurement ablation); 0 = lower triangle
  int ksplit;         // Gram only: > 1 = K cut into ksplit slices, summed by a second launch
  int pad_;
  float* part;        // ksplit > 1: kPartialFloats floats per (tile, slice), tile-major
};
static_assert(sizeof(Segment) == 48, "Segment layout");

// One fp32 partial product of a K slice: a 256 x 256 tile, or a small 128 x 128 one.
constexpr int kPartialFloats = 256 * 256;
constexpr int kSmallPartialFloats = kSmallTile * kSmallTile;

// Per-matrix scalars produced by the norm reduction.
struct alignas(16) MatScale {
  float c;      // 1 / (||Y|| + eps)
  float c2;     // c * c
  float norm;   // ||Y||
  float pad_;
};

constexpr int kMaxSegments = 64;

// Memory reached through descriptor fields is device (global) memory.  Saying
// so makes the compiler emit global_* instead of flat_* accesses: flat ones
// are counted by the LDS wait counter as well, so with flat stores in flight
// every wait for an LDS read would also wait for those stores to land.
template <typename T> using gptr = __attribute__((address_space(1))) T*;
typedef float f32v4 __attribute__((ext_vector_type(4)));  // builtin vector: copies through gptr
#if defined(__HIPCC__)
template <typename T> __device__ __forceinline__ gptr<T> gmem(T* p) { return (gptr<T>)p; }
#endif

}  // namespace dmuon
