// MFMA contraction kernels for one Newton-Schulz step on gfx950.
//
// One step of the cubic map (DMuon blog post, "Muon 核心：Newton-Schulz 迭代":
// G <- 1.5 G - 0.5 G G^T G, evaluated as two products, "代码实现") is two
// launches over every matrix of the batch:
//
//   syrk_kernel    A = alpha * X X^T      lower-triangle 256x256 tiles only; each
//                                         off-diagonal tile is also stored
//                                         transposed into the upper triangle, and
//                                         a diagonal tile computes only its MFMA
//                                         blocks on or below the diagonal and
//                                         stores the others as their transposes.
//   ns_gemm_kernel X <- g * (c0 X + c1 A X)    fused epilogue (blog's cubic map:
//                                         c0 = 1.5, c1 = -0.5); on the last step
//                                         it writes the update into the caller's
//                                         parameters (p -= lr * s * X) or output.
//
// A three-term map X <- c0 X + c1 A X + c2 A^2 X (custom coefficients, the
// training guide's NewtonSchulz object) adds one launch per step: syrk_kernel
// in square mode forms B = c2 A A + c1 A (A symmetric, so A A = A A^T, again
// on lower-triangle tiles), and ns_gemm_kernel then uses B with c1 = 1.
//
// Both are the block product C[i,j] = sum_k P[i,k] Q[k,j] with P K-contiguous.
// The Gram takes Q = X^T, i.e. Q's columns are rows of X, also K-contiguous
// (P = X).  The update takes P = A and Q = X read row-major: its stages land in
// LDS as K rows of 256 columns, and transposing LDS reads
// (ds_read_b64_tr_b16; fp32: single-word reads) hand each lane the
// K-consecutive values the MFMA expects.  Each 512-thread workgroup computes a 256x256
// tile; its eight waves form a 2 x 4 grid of 128x64 blocks, each 8x4 blocks of
// v_mfma_f32_16x16x32_bf16 (bf16) or 4x2 blocks of v_mfma_f32_32x32x2_f32
// (fp32), two waves per SIMD.  K advances 128 bytes per stage (64 bf16 / 32 fp32) through a
// double-buffered, XOR-swizzled LDS tile (2 x 64 KB) that global_load_lds
// fills directly (no register staging) while the current stage is multiplied;
// fragment reads and loads are issued one or two at a time between the MFMAs
// so that no burst of LDS or memory instructions stalls the matrix pipe.
//
// All device memory reached through descriptor pointers is accessed with
// global (not flat) instructions; see gmem().
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace dmuon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_ptr;

constexpr int kStageBytes = 65536;   // P (32 KB) + Q (32 KB)
constexpr int kOperandBytes = 32768; // 256 rows x 128 bytes

template <int DT> struct Elem;
template <> struct Elem<kBF16> { using T = __bf16; static constexpr int kBytes = 2; };
template <> struct Elem<kF32> { using T = float; static constexpr int kBytes = 4; };

__device__ __forceinline__ float to_f32(__bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return static_cast<T>(v); }

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8).  Within a segment of n tiles whose blocks start at t0, give each XCD
// one contiguous n/8 share of the segment's tile order, so neighbouring tiles
// (which share operand panels) meet in the same L2.  Returns the tile index
// for block t0 + local; a bijection on [0, n).
__device__ __forceinline__ int xcd_share(int local, int n, int t0) {
  const int x = (t0 + local) & 7;
  int off = 0, first_x = 0;
#pragma unroll
  for (int y = 0; y < 8; ++y) {
    const int f = (y - (t0 & 7) + 8) & 7;  // first local index placed on XCD y
    const int cnt = f < n ? (n - f + 7) >> 3 : 0;
    if (y < x) off += cnt;
    if (y == x) first_x = f;
  }
  return off + ((local - first_x) >> 3);
}

// Tile index for block t0 + local of a segment of n tiles, by rounds of 256:
// in round c, the XCD that runs local indices = f (mod 8) takes the 32
// consecutive tiles 256 c + 32 f .. 256 c + 32 f + 31 of the segment's tile
// order, one per CU of the XCD.  Within an XCD the resident tiles are a
// compact block of neighbours (shared operand panels in its L2), and at any
// moment all eight XCDs work in the same 256-tile window, i.e. on the same
// one or two matrices, whose panels the memory-side cache that every XCD
// reads through can then hold.  Tiles after the last whole round are split
// as in xcd_share.  A bijection on [0, n).
__device__ __forceinline__ int xcd_tile(int local, int n, int t0) {
  const int base = (n >> 8) << 8;
  if (local < base) return (((local >> 8) << 3) + (local & 7)) * 32 + ((local >> 3) & 31);
  return base + xcd_share(local - base, n - base, t0);
}

struct TileRef {
  int mat;     // NS descriptor index
  int bi;      // tile row
  int bj;      // tile col
  int kdim;
  int full;    // Gram segment computing every tile (no mirror)
  int ksplit;  // K slices of a split Gram segment (1: whole K in one block)
  int slice;   // this block's K slice (product launch of a split segment)
  float* part; // the tile's first partial product (split segments)
};

// reduce: the block is one tile of a split segment's summing launch (one
// block per tile); otherwise a split segment has one block per (tile, slice),
// the slices of a tile adjacent.  part_floats: the size of one partial product.
__device__ __forceinline__ TileRef locate(const SegTable& st, int block, bool lower, bool reduce = false,
                                          int part_floats = kPartialFloats) {
  int si = 0;
  while (si + 1 < st.nseg && st.seg[si + 1].tile0 <= block) ++si;
  const Segment& sg = st.seg[si];
  int local = xcd_tile(block - sg.tile0, sg.ntiles, sg.tile0);
  TileRef r;
  r.ksplit = sg.ksplit > 1 ? sg.ksplit : 1;
  r.slice = 0;
  if (r.ksplit > 1 && !reduce) {
    r.slice = local % r.ksplit;
    local /= r.ksplit;
  }
  r.part = r.ksplit > 1 ? sg.part + static_cast<long>(local) * r.ksplit * part_floats : nullptr;
  r.mat = sg.mat0 + local / sg.tiles_per_mat;
  const int t = local % sg.tiles_per_mat;
  r.kdim = sg.kdim;
  r.full = sg.full;
  if (lower && !sg.full) {
    // t -> (bi, bj), bj <= bi.  Groups of kTriGroupRows tile rows, each walked
    // column by column, take the same index ranges as the rows do in
    // row-major order: find t's row-major row, then place t in its group.
    constexpr int kTriGroupRows = 4;
    int row = static_cast<int>((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
    while ((row + 1) * (row + 2) / 2 <= t) ++row;
    while (row * (row + 1) / 2 > t) --row;
    const int r0 = row - row % kTriGroupRows;
    const int h = min(sg.tm - r0, kTriGroupRows);
    int tl = t - r0 * (r0 + 1) / 2;
    if (tl < h * r0) {
      // columns left of the group's own triangle: h tiles each
      r.bi = r0 + tl % h;
      r.bj = tl / h;
    } else {
      // the group's triangle, column bj holding rows bj .. r0 + h - 1
      tl -= h * r0;
      int bj = r0;
      while (tl >= r0 + h - bj) {
        tl -= r0 + h - bj;
        ++bj;
      }
      r.bi = bj + tl;
      r.bj = bj;
    }
  } else {
    // groups of kGroupRows tile rows, walked column by column, so the tiles
    // resident at one time share few P row panels and Q column panels
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

typedef __attribute__((address_space(3))) char* lds_cptr_t;

// Byte address of a __shared__ location in the LDS aperture.
__device__ __forceinline__ uint32_t lds_address(char* p) {
  return static_cast<uint32_t>(reinterpret_cast<size_t>((lds_cptr_t)p));  // address-space cast
}

// A workgroup-uniform pointer moved into SGPRs (it is computed from the block
// index and descriptor fields, but not always provably uniform to the compiler).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// global_load_lds_dwordx4: 16 bytes from base + voff (per lane) to
// LDS[lds_dst + 16 * lane].  Issued through asm so the compiler's wait-count
// pass does not treat it as an LDS operation of unknown completion order
// (which would force a full LDS wait before every fragment use); callers wait
// with an explicit vmcnt(0) and a barrier before reading the data.  M0 is set
// here and used by nothing else in these kernels; s_nop covers the M0 hazard.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
               "s"(lds_dst)
               : "memory");
}

// The same with a full 64-bit source address per lane (no scalar base), as a
// streaming (non-temporal) access: used for data read once per launch.
__device__ __forceinline__ void lds_dma16_addr_nt(const void* src, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds_dst)
               : "memory");
}

template <int N> __device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Wave grid of a 256x256 tile: 2 waves along M (128 rows each) and
// kWaves / 2 along N; each wave owns kBM x kBN blocks of 32x32 (the fp32 MFMA
// shape; bf16 splits each into 2 x 2 blocks of 16x16).
template <int kWaves>
struct WaveGrid {
  static constexpr int kThreadsPerBlock = 64 * kWaves;
  static constexpr int kWN = kWaves / 2;
  static constexpr int kBM = 4;                    // 128 rows
  static constexpr int kBN = 256 / kWN / 32;       // 32-column blocks per wave
  static constexpr int kLoadsPerOperand = 256 / kWaves / 8;  // 8-row wave loads per operand
};

// Accumulate the 256x256 tile of P * Q^T into acc: the fp32 kernels, on
// v_mfma_f32_32x32x2_f32 (bf16 runs block_product16 below).  P0 points at the first
// row of the 256-row P panel, rows K-contiguous, pitch ldp_bytes.  Q comes in
// one of two layouts:
//   QN == false: like P, 256 rows (j) with K contiguous (the Gram: rows of X);
//   QN == true:  K rows of 256 columns (j) with j contiguous (the update: X
//                itself); Q0 points at row 0, column j0, pitch ldq_bytes.
// kbytes is the contraction length in bytes (a multiple of 256 elements).
// before_last_stage(i), i = 0 .. 2 * 256 / kWaves / 8 - 1, issues the
// caller's own loads into the first 64 KB of LDS while the last stage is
// multiplied (one per call, spread between MFMAs).  after_last_barrier() runs
// once every wave has read its last operand fragment: from then on the caller
// owns all of the LDS, while the final MFMAs are still in flight.
// kMask: bit mi * kBN + ni set when the caller needs the wave's 32 x 32 block
// (mi, ni); the wave runs only those blocks' MFMAs and reads only the
// fragments they use, leaving the other accumulators as they are.  Every
// wave, even one with no block to compute, still issues its share of every
// stage's loads and joins every barrier.
//
// Global -> LDS: global_load_lds_dwordx4 writes lane l's 16 bytes to
// LDS[M0 + 16 l], so one wave instruction fills 1 KB of a stage.  Each lane
// fetches the source chunk that belongs in its slot of the XOR-swizzled
// layout the fragment reads expect, so there is no VGPR staging.
template <int DT, int kWaves, bool QN, unsigned kMask = 0xFFu, typename BeforeLastStage, typename AfterLastBarrier>
__device__ __forceinline__ void block_product(const char* __restrict__ P0, int ldp_bytes,
                                              const char* __restrict__ Q0, int ldq_bytes, int kbytes, char* lds,
                                              f32x16 (&acc)[4][WaveGrid<kWaves>::kBN],
                                              BeforeLastStage&& before_last_stage,
                                              AfterLastBarrier&& after_last_barrier) {
  static_assert(DT == kF32, "bf16 products run block_product16");
  using G = WaveGrid<kWaves>;
  constexpr int kBN = G::kBN;
  constexpr int kRowsPerWave = 256 / kWaves;
  constexpr int EB = 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / G::kWN, wc = wave % G::kWN;
  const int li = lane & 31, lh = lane >> 5;

  // K-contiguous operands: row r of a stage stores logical 16-byte chunk c at
  // slot c ^ swz(r) with swz(r) = (r & 7) ^ ((r >> 3) & 1): the 16 lanes an
  // LDS cycle serves for ds_read_b128 (rows r..r+15, 64 banks) and any 8
  // consecutive rows then hit distinct banks.  The wave's 8-row load groups
  // start at multiples of 8, so for load group u the swizzle is lrow ^ (u & 1).
  P0 = uniform_ptr(P0);
  Q0 = uniform_ptr(Q0);
  const int lrow = lane >> 3;                    // row within an 8-row group
  const int lchunk0 = (lane & 7) ^ lrow;         // source chunk, even load groups
  const int lchunk1 = lchunk0 ^ 1;               // odd load groups
  const uint32_t rp = static_cast<uint32_t>((wave * kRowsPerWave + lrow) * ldp_bytes);
  const uint32_t offp0 = rp + lchunk0 * 16, offp1 = rp + lchunk1 * 16;
  const uint32_t grp_p = static_cast<uint32_t>(8 * ldp_bytes);

  // Q offsets.  K-contiguous: as P.  Column-contiguous (QN): a stage holds
  // kQRows = 32 rows of 256 fp32 (the same K as a 128-byte K step); wave w
  // fills rows of KB blocks 4 w .. 4 w + 3.  Row r of the stage stores logical
  // chunk c at slot c ^ qswz(r), qswz(r) = 8 ((r >> 2) & 1): the 4-byte reads
  // of rows r and r + 4, 128 bytes each, hit distinct banks.
  constexpr int kQRowBytes = 256 * EB;
  constexpr int kQRows = kOperandBytes / kQRowBytes;   // K rows per stage
  constexpr int kQRowsPerKB = 1024 / kQRowBytes;       // rows per 1 KB wave load
  uint32_t offq0, offq1, grp_q;
  if constexpr (QN) {
    const int sub = lane / (64 / kQRowsPerKB);          // row within the KB block
    const int pc = lane % (64 / kQRowsPerKB);           // physical chunk in the row
    const int r0 = wave * 4 * kQRowsPerKB + sub;        // rows of load u: r0 + u * kQRowsPerKB
    auto qswz = [](int r) { return 8 * ((r >> 2) & 1); };
    offq0 = static_cast<uint32_t>(r0 * ldq_bytes + ((pc ^ qswz(r0)) << 4));
    offq1 = static_cast<uint32_t>((r0 + kQRowsPerKB) * ldq_bytes + ((pc ^ qswz(r0 + kQRowsPerKB)) << 4)) -
            static_cast<uint32_t>(kQRowsPerKB * ldq_bytes);
    grp_q = static_cast<uint32_t>(kQRowsPerKB * ldq_bytes);
  } else {
    const uint32_t rq = static_cast<uint32_t>((wave * kRowsPerWave + lrow) * ldq_bytes);
    offq0 = rq + lchunk0 * 16;
    offq1 = rq + lchunk1 * 16;
    grp_q = static_cast<uint32_t>(8 * ldq_bytes);
  }
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_address(lds) + wave * kRowsPerWave * 128);

  // fragment reads: row (block * 32 + li), logical chunk 2 s + lh
  const int frag_row = li * 128;
  const int sw = (li & 7) ^ ((li >> 3) & 1);
  // QN fragment offsets (bytes within the Q region of a stage, without the
  // sub-step's row offset), one per 32-column block x of the wave
  int qfrag[kBN];
  if constexpr (QN) {
#pragma unroll
    for (int x = 0; x < kBN; ++x) {
      // element e of sub-step s: row 8 s + 4 lh + e, column 32 J + li
      const int J = wc * kBN + x;
      qfrag[x] = 4 * lh * kQRowBytes + ((8 * (J ^ lh) + (li >> 2)) << 4) + 4 * (li & 3);
    }
  }

  using Frag = f32x4;
  Frag fa[2][4], fb[2][kBN];
  constexpr int kMfma = 4 * kBN;                    // MFMA blocks per sub-step
  constexpr int kReads = 4 + kBN;                   // fragment reads per sub-step
  constexpr int kDma = 2 * G::kLoadsPerOperand;     // DMA loads per stage
  auto read_q = [&](int stage, int s, int rs, int x) {
    const char* qbase = lds + stage * kStageBytes + kOperandBytes;
    if constexpr (!QN) {
      const int co = (((2 * s + lh) ^ sw) << 4);
      fb[rs][x] = *reinterpret_cast<const Frag*>(qbase + frag_row + co + (wc * kBN + x) * 32 * 128);
    } else {
      const char* b = qbase + qfrag[x] + 8 * s * kQRowBytes;
#pragma unroll
      for (int e = 0; e < 4; ++e) fb[rs][x][e] = *reinterpret_cast<const float*>(b + e * kQRowBytes);
    }
  };
  // read i of a sub-step, in the order the MFMAs need them: fb[0], fa[0], fb[1..], fa[1..]
  // fragments some needed block uses: P row block mi, Q column block ni
  constexpr unsigned kRowBits = (1u << kBN) - 1u;
  auto p_used = [](int mi) { return ((kMask >> (mi * kBN)) & kRowBits) != 0u; };
  auto q_used = [](int ni) {
    unsigned any = 0u;
    for (int mi = 0; mi < 4; ++mi) any |= (kMask >> (mi * kBN + ni)) & 1u;
    return any != 0u;
  };
  auto read_one = [&](int stage, int s, int rs, int i) {
    if (i == 0 || (i >= 2 && i < kBN + 1)) {
      if (!q_used(i == 0 ? 0 : i - 1)) return;
    } else if (!p_used(i == 1 ? 0 : i - kBN)) {
      return;
    }
    const int co = (((2 * s + lh) ^ sw) << 4);
    const char* base = lds + stage * kStageBytes + frag_row + co;
    if (i == 0) read_q(stage, s, rs, 0);
    else if (i == 1) fa[rs][0] = *reinterpret_cast<const Frag*>(base + (wr * 4) * 32 * 128);
    else if (i < kBN + 1) read_q(stage, s, rs, i - 1);
    else fa[rs][i - kBN] = *reinterpret_cast<const Frag*>(base + (wr * 4 + i - kBN) * 32 * 128);
  };
  // DMA load i of the stage starting at K byte offset kb (K-contiguous units)
  auto dma_one = [&](int stage, int kb, int i) {
    const uint32_t dp = lds_wave + stage * kStageBytes;
    const int u = i >> 1;
    if ((i & 1) == 0) {
      lds_dma16(P0, ((u & 1) ? offp1 : offp0) + u * grp_p + kb, dp + u * 1024);
    } else if constexpr (QN) {
      const char* qk = Q0 + static_cast<long>(kb >> 7) * kQRows * static_cast<long>(ldq_bytes);
      lds_dma16(qk, ((u & 1) ? offq1 : offq0) + u * grp_q, dp + kOperandBytes + u * 1024);
    } else {
      lds_dma16(Q0, ((u & 1) ? offq1 : offq0) + u * grp_q + kb, dp + kOperandBytes + u * 1024);
    }
  };
  auto mfma_one = [&](int rs, int j) {
    if (((kMask >> j) & 1u) == 0u) return;
    const int mi = j / kBN, ni = j % kBN;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[rs][ni][e], fa[rs][mi][e], acc[mi][ni], 0, 0, 0);
  };
  // One sub-step: the MFMAs of register slot rs, with the next sub-step's
  // fragment reads (from (rstage, rsub) into slot rs ^ 1) and nd DMA loads
  // (dma(0) .. dma(nd - 1)) spread between them, each group pinned in place so
  // no burst of LDS or memory issues stalls the MFMA stream.
  auto substep = [&](int rs, int rstage, int rsub, auto&& dma, int nd) {
#pragma unroll
    for (int j = 0; j < kMfma; ++j) {
      mfma_one(rs, j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = j * kReads / kMfma; i < (j + 1) * kReads / kMfma; ++i) read_one(rstage, rsub, rs ^ 1, i);
#pragma unroll
      for (int i = j * nd / kMfma; i < (j + 1) * nd / kMfma; ++i) dma(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto no_dma = [](int) {};

  // Pipeline: stage kt is multiplied from buffer kt & 1 while stage kt + 1
  // lands in the other buffer.  Stage kt + 2's loads go into buffer kt & 1
  // once the barrier after sub-step 2 has retired every read of it, spread
  // over sub-step 3 of stage kt; they have until the barrier after sub-step 2
  // of stage kt + 1 to land.  The buffer stage nk - 2 frees receives the
  // caller's early loads instead (before_last_stage(0 .. kDma - 1)).  nk is
  // even and at least 4: every contraction extent is a multiple of 256.
  const int nk = kbytes / 128;
#pragma unroll
  for (int i = 0; i < kDma; ++i) dma_one(0, 0, i);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kDma; ++i) dma_one(1, 128, i);
#pragma unroll
  for (int i = 0; i < kReads; ++i) read_one(0, 0, 0, i);
  __builtin_amdgcn_sched_barrier(0);
  for (int kt = 0; kt < nk - 2; ++kt) {
    const int c = kt & 1;
    substep(0, c, 1, no_dma, 0);
    substep(1, c, 2, no_dma, 0);
    substep(0, c, 3, no_dma, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    substep(1, c ^ 1, 0, [&](int i) { dma_one(c, (kt + 2) * 128, i); }, kDma);
  }
  // stage nk - 2: buffer 0 is free after its barrier
  substep(0, 0, 1, no_dma, 0);
  substep(1, 0, 2, no_dma, 0);
  substep(0, 0, 3, no_dma, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  substep(1, 1, 0, before_last_stage, kDma);
  // final stage: no more loads; after its barrier nothing reads the operand
  // buffers again, so the caller may start filling LDS while the last
  // sub-step's MFMAs run
  substep(0, 1, 1, no_dma, 0);
  substep(1, 1, 2, no_dma, 0);
  substep(0, 1, 3, no_dma, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  after_last_barrier();
#pragma unroll
  for (int j = 0; j < kMfma; ++j) mfma_one(1, j);
}

// Eight waves (two per SIMD) in a 2 x 4 grid of 128 x 64 blocks.  The load
// maps and the update epilogue's vmcnt counts are written for this count.
constexpr int kWaves = 8;
// The bf16 form of block_product on v_mfma_f32_16x16x32_bf16: each wave's
// 128 x 64 block is 8 x 4 blocks of 16 x 16, acc16[mi][ni] holding
//   C[16 mi + (lane & 15)][16 ni + 4 (lane >> 4) + q],  q = 0..3,
// and K advances 32 per MFMA.  At the power limit an MFMA-only loop on random
// bf16 operands sustains 11% more flops with this shape than with 32x32x16
// (it moves fewer accumulator registers per flop).  Loads, stages, barriers
// and hooks are those of block_product; a 64-deep stage is two sub-steps of
// 32, each split into two quarter-steps by P row-block halves.  Fragment reads (k = (0, 2, 1, 3)[l >> 4], the stage octet lane l's K
// octet comes from): P (and a K-contiguous Q) lane l reads 16 bytes of row
// 16 blk + (l & 15), logical chunk 4 s + k.  A row-major Q (QN) comes in
// through two ds_read_b64_tr_b16 per fragment: in each 16-lane group,
// lane 4 t + a points at K row 32 s + 8 k + 4 r + t (read r),
// columns 16 blk + 4 a .. + 3, and receives column 16 blk + (l & 15) of those
// four rows.  The row-major stage's swizzle qswz(r) = 4 (r & 3) ^ 2 ((r >> 4) & 1)
// keeps the two groups a 64-bit read serves together (lanes 0..31: rows 16
// apart) in distinct banks.
// kMask: bit 4 mi + ni set when block (mi, ni) is needed.
template <bool QN, unsigned kMask = 0xFFFFFFFFu, typename BeforeLastStage, typename AfterLastBarrier>
__device__ __forceinline__ void block_product16(const char* __restrict__ P0, int ldp_bytes,
                                                const char* __restrict__ Q0, int ldq_bytes, int kbytes, char* lds,
                                                f32x4 (&acc)[8][4], BeforeLastStage&& before_last_stage,
                                                AfterLastBarrier&& after_last_barrier) {
  using G = WaveGrid<8>;
  constexpr int kRowsPerWave = 256 / 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / G::kWN, wc = wave % G::kWN;

  P0 = uniform_ptr(P0);
  Q0 = uniform_ptr(Q0);
  // DMA source offsets, as in block_product
  const int lrow = lane >> 3;
  const int lchunk0 = (lane & 7) ^ lrow;
  const int lchunk1 = lchunk0 ^ 1;
  const uint32_t rp = static_cast<uint32_t>((wave * kRowsPerWave + lrow) * ldp_bytes);
  const uint32_t offp0 = rp + lchunk0 * 16, offp1 = rp + lchunk1 * 16;
  const uint32_t grp_p = static_cast<uint32_t>(8 * ldp_bytes);
  constexpr int kQRowBytes = 512;                     // 256 bf16 columns
  constexpr int kQRows = kOperandBytes / kQRowBytes;  // 64 K rows per stage
  constexpr int kQRowsPerKB = 2;
  static_assert(kQRows == 64, "row-major stage");
  uint32_t offq0, offq1, grp_q;
  if constexpr (QN) {
    // wave w fills K rows 8 w .. 8 w + 7 (KB blocks 4 w .. 4 w + 3)
    const int sub = lane / 32, pc = lane % 32;
    const int r0 = wave * 4 * kQRowsPerKB + sub;
    auto qswz = [](int r) { return (4 * (r & 3)) ^ (2 * ((r >> 4) & 1)); };
    offq0 = static_cast<uint32_t>(r0 * ldq_bytes + ((pc ^ qswz(r0)) << 4));
    offq1 = static_cast<uint32_t>((r0 + kQRowsPerKB) * ldq_bytes + ((pc ^ qswz(r0 + kQRowsPerKB)) << 4)) -
            static_cast<uint32_t>(kQRowsPerKB * ldq_bytes);
    grp_q = static_cast<uint32_t>(kQRowsPerKB * ldq_bytes);
  } else {
    const uint32_t rq = static_cast<uint32_t>((wave * kRowsPerWave + lrow) * ldq_bytes);
    offq0 = rq + lchunk0 * 16;
    offq1 = rq + lchunk1 * 16;
    grp_q = static_cast<uint32_t>(8 * ldq_bytes);
  }
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_address(lds) + wave * kRowsPerWave * 128);

  // Lane group lq = lane >> 4 holds the MFMA's K octet lq; it reads the
  // stage's octet lk = (0, 2, 1, 3)[lq] of the sub-step, the same for both
  // operands, so each K index is still summed once.  ds_read_b128 serves
  // lanes l and l + 32 together: with this order they read adjacent chunks
  // of a row, which the swizzle keeps in distinct banks.
  // K-contiguous fragment reads: row 16 blk + (lane & 15), chunk 4 s + lk
  const int l16 = lane & 15, lq = lane >> 4;
  const int lk = ((lq & 1) << 1) | (lq >> 1);
  const int frag_row = l16 * 128;
  const int sw = (l16 & 7) ^ ((l16 >> 3) & 1);
  // QN fragment offsets within the Q region (without the sub-step's rows), per block ni
  int qfrag[4];
  if constexpr (QN) {
    const int t = (lane >> 2) & 3, a = lane & 3;
    const int qs = (4 * t) ^ (2 * ((lk >> 1) & 1));
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int ch = 8 * wc + 2 * x + (a >> 1);
      qfrag[x] = (8 * lk + t) * kQRowBytes + ((ch ^ qs) << 4) + 8 * (a & 1);
    }
  }

  // blocks and fragments some needed block uses
  auto p_used = [](int mi) { return ((kMask >> (4 * mi)) & 0xFu) != 0u; };
  auto q_used = [](int ni) { return ((kMask >> ni) & 0x11111111u) != 0u; };
  // A 64-deep stage is four quarter-steps of 16 MFMAs: (sub-step s, half h)
  // multiplies P row blocks 4 h .. 4 h + 3 by Q column blocks 0..3 at K
  // 32 s .. 32 s + 31.  fb[s] holds sub-step s's Q fragments, fa[h] half h's
  // P fragments; each quarter-step reads what the next one needs:
  //   q0 (s0 h0): fa[1] <- sub 0 half 1
  //   q1 (s0 h1): fb[1] <- sub 1, fa[0] <- sub 1 half 0
  //   q2 (s1 h0): fa[1] <- sub 1 half 1
  //   q3 (s1 h1): fb[0], fa[0] <- the next stage's sub 0 (other buffer)
  bf16x8 fa[2][4], fb[2][4];
  constexpr int kDma = 2 * G::kLoadsPerOperand;     // DMA loads per stage
  auto read_q = [&](int stage, int sub, int x) {
    if (!q_used(x)) return;
    const char* qbase = lds + stage * kStageBytes + kOperandBytes;
    if constexpr (!QN) {
      const int co = (((4 * sub + lk) ^ sw) << 4);
      fb[sub][x] = *reinterpret_cast<const bf16x8*>(qbase + frag_row + co + (wc * 4 + x) * 16 * 128);
    } else {
      const char* b = qbase + qfrag[x] + 32 * sub * kQRowBytes;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<lds_bf16x4_ptr>((lds_cptr_t)b));
      const bf16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<lds_bf16x4_ptr>((lds_cptr_t)(b + 4 * kQRowBytes)));
      fb[sub][x] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto read_p = [&](int stage, int sub, int h, int i) {
    if (!p_used(4 * h + i)) return;
    const int co = (((4 * sub + lk) ^ sw) << 4);
    fa[h][i] = *reinterpret_cast<const bf16x8*>(lds + stage * kStageBytes + frag_row + co +
                                                (wr * 8 + 4 * h + i) * 16 * 128);
  };
  auto dma_one = [&](int stage, int kb, int i) {
    const uint32_t dp = lds_wave + stage * kStageBytes;
    const int u = i >> 1;
    if ((i & 1) == 0) {
      lds_dma16(P0, ((u & 1) ? offp1 : offp0) + u * grp_p + kb, dp + u * 1024);
    } else if constexpr (QN) {
      const char* qk = Q0 + static_cast<long>(kb >> 7) * kQRows * static_cast<long>(ldq_bytes);
      lds_dma16(qk, ((u & 1) ? offq1 : offq0) + u * grp_q, dp + kOperandBytes + u * 1024);
    } else {
      lds_dma16(Q0, ((u & 1) ? offq1 : offq0) + u * grp_q + kb, dp + kOperandBytes + u * 1024);
    }
  };
  auto mfma_one = [&](int s, int h, int j) {
    const int mi = 4 * h + j / 4, ni = j % 4;
    if (((kMask >> (4 * mi + ni)) & 1u) == 0u) return;
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[s][ni], fa[h][j / 4], acc[mi][ni], 0, 0, 0);
  };
  // One quarter-step: its 16 MFMAs with nr reads (rd(0) .. rd(nr - 1)) and nd
  // DMA loads between them, each group pinned in place.  The DMA loads are
  // spread over all 16 MFMAs.  early: the reads go one after each of the
  // first nr MFMAs, so they land well before the quarter-step ends (and
  // before the barrier after quarter-step 2); otherwise they are spread too.
  // The main loop takes them early: its stages ran 0.3% (update) and 0.9%
  // (Gram) faster so in same-box comparisons; the two peeled stages keep
  // the spread order except before their barrier.
  auto quarter = [&](int s, int h, auto&& rd, int nr, auto&& dma, int nd, bool early = false) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      mfma_one(s, h, j);
      __builtin_amdgcn_sched_barrier(0);
      if (early) {
        if (j < nr) rd(j);
      } else {
#pragma unroll
        for (int i = j * nr / 16; i < (j + 1) * nr / 16; ++i) rd(i);
      }
#pragma unroll
      for (int i = j * nd / 16; i < (j + 1) * nd / 16; ++i) dma(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto no_dma = [](int) {};
  // the reads each quarter-step issues; the next stage's sub-step 0 comes
  // from buffer nc: Q fragments first, in the order the MFMAs use them
  auto rd_q0 = [&](int c) { return [&, c](int i) { read_p(c, 0, 1, i); }; };
  auto rd_q1 = [&](int c) { return [&, c](int i) { if (i < 4) read_q(c, 1, i); else read_p(c, 1, 0, i - 4); }; };
  auto rd_q2 = [&](int c) { return [&, c](int i) { read_p(c, 1, 1, i); }; };
  auto rd_q3 = [&](int nc) { return [&, nc](int i) { if (i < 4) read_q(nc, 0, i); else read_p(nc, 0, 0, i - 4); }; };
  auto no_rd = [](int) {};

  // Pipeline: stage kt is multiplied from buffer kt & 1 while stage kt + 1
  // lands in the other buffer.  After quarter-step 2 every read of buffer
  // kt & 1 has been issued; the barrier retires them, and quarter-step 3
  // issues stage kt + 2's loads into that buffer, which have until the barrier
  // after the next stage's quarter-step 2 to land.  The buffer stage nk - 2
  // frees receives the caller's early loads instead (before_last_stage).
  const int nk = kbytes / 128;
#pragma unroll
  for (int i = 0; i < kDma; ++i) dma_one(0, 0, i);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kDma; ++i) dma_one(1, 128, i);
#pragma unroll
  for (int i = 0; i < 8; ++i) rd_q3(0)(i);
  __builtin_amdgcn_sched_barrier(0);
  for (int kt = 0; kt < nk - 2; ++kt) {
    const int c = kt & 1;
    quarter(0, 0, rd_q0(c), 4, no_dma, 0, true);
    quarter(0, 1, rd_q1(c), 8, no_dma, 0, true);
    quarter(1, 0, rd_q2(c), 4, no_dma, 0, true);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    quarter(1, 1, rd_q3(c ^ 1), 8, [&](int i) { dma_one(c, (kt + 2) * 128, i); }, kDma, true);
  }
  // stage nk - 2: buffer 0 is free after its barrier
  quarter(0, 0, rd_q0(0), 4, no_dma, 0);
  quarter(0, 1, rd_q1(0), 8, no_dma, 0);
  quarter(1, 0, rd_q2(0), 4, no_dma, 0, true);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  quarter(1, 1, rd_q3(1), 8, before_last_stage, kDma);
  // final stage: no more loads; after its barrier nothing reads the operand
  // buffers again, so the caller may start filling LDS while the last
  // quarter-step's MFMAs run
  quarter(0, 0, rd_q0(1), 4, no_dma, 0);
  quarter(0, 1, rd_q1(1), 8, no_dma, 0);
  quarter(1, 0, rd_q2(1), 4, no_dma, 0, true);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  after_last_barrier();
  quarter(1, 1, no_rd, 0, no_dma, 0);
}


using Grid = WaveGrid<kWaves>;
constexpr int kBN = Grid::kBN;
constexpr int kThreads = Grid::kThreadsPerBlock;

// Per-wave accumulators: bf16 on 16 x 16 MFMA blocks (block_product16), fp32
// on 32 x 32 ones (block_product).  Both are 128 floats per lane.
template <int DT> struct AccOf { using type = f32x16[4][kBN]; };
template <> struct AccOf<kBF16> { using type = f32x4[8][4]; };
template <int DT> using Acc = typename AccOf<DT>::type;
template <int DT> __device__ __forceinline__ void zero_acc(Acc<DT>& acc) {
  if constexpr (DT == kBF16) {
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{};
  } else {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < kBN; ++ni) acc[mi][ni] = f32x16{};
  }
}

// ---------------------------------------------------------------- epilogue
// The MFMAs take (Q, P) so each accumulator block holds the transposed
// product: lane (li, lh), register 4 g + q of block (mi, ni) is
//   C[32 mi + li][32 (wc kBN + ni) + 8 g + 4 lh + q]
// (rows relative to the wave's 128-row half), i.e. four consecutive columns of
// one row.  The Gram epilogue stages one 128 x 256 fp32 half-tile at a time
// in the 128 KB of LDS the operand stages no longer need, then writes every
// output with 16-byte lanes: rows for row-major outputs, 8-row column
// segments for transposed ones.  The update epilogue uses the same layout for
// its 64-row quarters, one 64 KB buffer each.
//
// Staging layout: 16-byte chunk c (0..63) of row r (0..127) lives at chunk
// c ^ swz(r), swz(r) = (r ^ (r >> 3)) & 63.  Conflict-free for the three
// patterns used: fragment stores (16 rows x one chunk), row reads (one row x
// 64 chunks) and column reads (rows 8 s + i, s = 0..15, four adjacent columns).
__device__ __forceinline__ int stage_off(int r, int c) { return r * 1024 + ((c ^ ((r ^ (r >> 3)) & 63)) << 4); }

__device__ __forceinline__ void stage_acc(char* lds, const f32x16 (&acc)[4][kBN], float scale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int cbase = (wave % Grid::kWN) * kBN * 8;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < kBN; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 v = make_float4(acc[mi][ni][4 * g] * scale, acc[mi][ni][4 * g + 1] * scale,
                                     acc[mi][ni][4 * g + 2] * scale, acc[mi][ni][4 * g + 3] * scale);
        *reinterpret_cast<float4*>(lds + stage_off(32 * mi + li, cbase + 8 * ni + 2 * g + lh)) = v;
      }
}

// The same from 16 x 16 blocks: lane l of block (mi, ni) holds row
// 16 mi + (l & 15), columns 16 ni + 4 (l >> 4) .. + 3 of the wave's block.
__device__ __forceinline__ void stage_acc(char* lds, const f32x4 (&acc)[8][4], float scale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cbase = (wave % Grid::kWN) * kBN * 8;
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const f32x4& a = acc[mi][ni];
      *reinterpret_cast<float4*>(lds + stage_off(16 * mi + (lane & 15), cbase + 4 * ni + (lane >> 4))) =
          make_float4(a[0] * scale, a[1] * scale, a[2] * scale, a[3] * scale);
    }
}

__device__ __forceinline__ float4 stage_ld4(const char* lds, int r, int c) {
  return *reinterpret_cast<const float4*>(lds + stage_off(r, c));
}
__device__ __forceinline__ void stage_st4(char* lds, int r, int c, float4 v) {
  *reinterpret_cast<float4*>(lds + stage_off(r, c)) = v;
}
// Column segment: rows 8 s .. 8 s + 7 of column col.
__device__ __forceinline__ void stage_col8(const char* lds, int s, int col, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = *reinterpret_cast<const float*>(lds + stage_off(8 * s + i, col >> 2) + (col & 3) * 4);
}

// 4 / 8 consecutive elements of T to and from fp32 (16-byte aligned vectors).
__device__ __forceinline__ void vst4(float* p, const float* v) {
  *reinterpret_cast<gptr<f32v4>>(gmem(p)) = f32v4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ void vst4(__bf16* p, const float* v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 x;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = static_cast<__bf16>(v[e]);
  *reinterpret_cast<gptr<bf16x4>>(gmem(p)) = x;
}
// Streaming (non-temporal) form, for the iterate an update epilogue writes: a
// whole batch's iterate is far larger than any cache, so nothing of it
// survives until the next launch reads it, and streaming it leaves the cached
// operand panels that concurrent tiles share in place.
__device__ __forceinline__ void vst4_nt(__bf16* p, const float* v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 x;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = static_cast<__bf16>(v[e]);
  __builtin_nontemporal_store(x, reinterpret_cast<gptr<bf16x4>>(gmem(p)));
}
__device__ __forceinline__ void vld4(const float* p, float* v) {
  const f32v4 x = *reinterpret_cast<gptr<const f32v4>>(gmem(p));
  v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
}
__device__ __forceinline__ void vld4(const __bf16* p, float* v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 x = *reinterpret_cast<gptr<const bf16x4>>(gmem(p));
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = static_cast<float>(x[e]);
}
__device__ __forceinline__ void vst8(float* p, const float* v) { vst4(p, v); vst4(p + 4, v + 4); }
__device__ __forceinline__ void vst8(__bf16* p, const float* v) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  bf16x8_t x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<__bf16>(v[e]);
  *reinterpret_cast<gptr<bf16x8_t>>(gmem(p)) = x;
}

// Last Newton-Schulz step: N consecutive elements of U at caller (orow,
// ocol0 ..) -> p <- p * decay - lr*s*U (+ update_out) or out = U, masked to
// the caller's shape; 4-element vectors where the row layout and pointers
// allow it.  decay = 1 - lr * weight_decay (exactly 1 without decay).
template <typename T, int N>
__device__ __forceinline__ void write_caller(const MatDesc& d, int mode, float step_lr, float decay, int orow,
                                             int ocol0, const float* u) {
  if (orow >= d.m) return;
  const long o = static_cast<long>(orow) * d.n + ocol0;
  T* p = static_cast<T*>(d.p) + o;
  float* upd = d.upd ? d.upd + o : nullptr;
#pragma unroll
  for (int h4 = 0; h4 < N; h4 += 4) {
    const int c = ocol0 + h4;
    if (d.vec_ok && c + 4 <= d.n) {
      float v[4];
      if (mode == kModeMuon) {
        vld4(p + h4, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(step_lr, u[h4 + e], v[e] * decay);
        vst4(p + h4, v);
        if (upd) vst4(upd + h4, u + h4);
      } else {
        vst4(p + h4, u + h4);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (c + e >= d.n) break;
        if (mode == kModeMuon) {
          gmem(p)[h4 + e] = static_cast<T>(fmaf(step_lr, u[h4 + e], static_cast<float>(gmem(p)[h4 + e]) * decay));
          if (upd) gmem(upd)[h4 + e] = u[h4 + e];
        } else {
          gmem(p)[h4 + e] = static_cast<T>(u[h4 + e]);
        }
      }
    }
  }
}

// A split Gram tile's partial product: thread tid's accumulator registers as
// float4 j = 4 (mi kBN + ni) + g at float4 index j * kThreads + tid, so each
// wave instruction moves 1 KB of consecutive memory and the summing launch
// reads back exactly the registers this thread held.
__device__ __forceinline__ void store_partial(float* part, const f32x16 (&acc)[4][kBN]) {
  f32v4* dst = reinterpret_cast<f32v4*>(part) + threadIdx.x;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < kBN; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc[mi][ni];
        *gmem(dst + ((mi * kBN + ni) * 4 + g) * kThreads) =
            f32v4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
      }
}

__device__ __forceinline__ void store_partial(float* part, const f32x4 (&acc)[8][4]) {
  f32v4* dst = reinterpret_cast<f32v4*>(part) + threadIdx.x;
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    const f32x4& a = acc[b >> 2][b & 3];
    *gmem(dst + b * kThreads) = f32v4{a[0], a[1], a[2], a[3]};
  }
}

__device__ __forceinline__ void add_partial(const float* part, f32x4 (&acc)[8][4]) {
  const f32v4* src = reinterpret_cast<const f32v4*>(part) + threadIdx.x;
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    const f32v4 v = *gmem(src + b * kThreads);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[b >> 2][b & 3][e] += v[e];
  }
}

__device__ __forceinline__ void add_partial(const float* part, f32x16 (&acc)[4][kBN]) {
  const f32v4* src = reinterpret_cast<const f32v4*>(part) + threadIdx.x;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < kBN; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32v4 v = *gmem(src + ((mi * kBN + ni) * 4 + g) * kThreads);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mi][ni][4 * g + e] += v[e];
      }
}

template <int DT>
__global__ __launch_bounds__(kThreads, 1) void syrk_kernel(const MatDesc* __restrict__ descs, SegTable st,
                                                          const MatScale* __restrict__ scales, int step,
                                                          int square, float cq, float cl, int reduce) {
  using T = typename Elem<DT>::T;
  constexpr int EB = Elem<DT>::kBytes;
  __shared__ __attribute__((aligned(16))) char lds[2 * kStageBytes];

  const TileRef tr = locate(st, blockIdx.x, true, reduce != 0);
  const MatDesc& d = descs[tr.mat];
  const int mp = d.mp, np = d.np;
  // Gram of the iterate (K = Np), or the square of the symmetric Gram matrix
  // (K = Mp) for the c2 A^2 term of a three-term map
  const char* xs = static_cast<const char*>(square ? d.a : ((step & 1) ? d.xs1 : d.xs0));
  const int kdim = square ? mp : np;
  const long ld = static_cast<long>(kdim) * EB;
  // a lower-triangle tile on the diagonal (a full-Gram launch computes every
  // tile whole)
  const bool diag = tr.bi == tr.bj && !tr.full;

  Acc<DT> acc;
  zero_acc<DT>(acc);

  if (!reduce) {
    // K slice of this block: all of K, or 1 / ksplit of it (a multiple of 256)
    const int klen = kdim / tr.ksplit;
    const char* p = xs + static_cast<long>(tr.bi) * kTile * ld + static_cast<long>(tr.slice) * klen * EB;
    const char* q = xs + static_cast<long>(tr.bj) * kTile * ld + static_cast<long>(tr.slice) * klen * EB;
    // A diagonal tile needs only its MFMA blocks on or below the block
    // diagonal: the epilogue writes the others as transposes.  Each wave runs
    // one of four patterns (Grid: 2 x 4 waves).  bf16, 16 x 16 blocks: block
    // (R, C) = (8 wr + mi, 4 wc + ni), needed when C <= R.  fp32, 32 x 32
    // blocks: (4 wr + mi, 2 wc + ni).
    static_assert(Grid::kWN == 4 && kBN == 2, "diagonal block patterns");
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int band = (wv % Grid::kWN) - 2 * (wv / Grid::kWN);   // wave column pair relative to its row band
    auto run = [&](auto mask) {
      if constexpr (DT == kBF16)
        block_product16<false, decltype(mask)::value>(p, ld, q, ld, klen * EB, lds, acc, [](int) {}, [] {});
      else
        block_product<DT, kWaves, false, decltype(mask)::value>(p, ld, q, ld, klen * EB, lds, acc, [](int) {},
                                                                [] {});
    };
    constexpr bool k16 = DT == kBF16;
    using All = std::integral_constant<unsigned, k16 ? 0xFFFFFFFFu : 0xFFu>;
    using OnDiag = std::integral_constant<unsigned, k16 ? 0xFFFFF731u : 0xFDu>;     // C <= R within the wave
    using RightOfDiag = std::integral_constant<unsigned, k16 ? 0xF7310000u : 0xD0u>;
    if (!diag || band < 0) run(All{});                  // below the diagonal
    else if (band == 0) run(OnDiag{});
    else if (band == 1) run(RightOfDiag{});
    else run(std::integral_constant<unsigned, 0u>{});   // above the diagonal
    if (tr.ksplit > 1) {
      store_partial(tr.part + static_cast<long>(tr.slice) * kPartialFloats, acc);
      return;
    }
  } else {
    // the tile's slices, summed in slice order
    for (int s = 0; s < tr.ksplit; ++s) add_partial(tr.part + static_cast<long>(s) * kPartialFloats, acc);
  }

  const float alpha = square ? cq : (step == 0 ? scales[tr.mat].c2 : 1.0f);
  T* a = static_cast<T*>(square ? d.b : d.a);
  const T* a_in = static_cast<const T*>(d.a);
  const int tid = threadIdx.x, wr = (tid >> 6) / Grid::kWN;
  const int Rt = tr.bi * kTile, Ct = tr.bj * kTile;
  const bool mirror = tr.bi != tr.bj && !tr.full;
  __syncthreads();  // operand stages are free
  // A diagonal tile holds its MFMA blocks on and below the block diagonal:
  // rows write only those, and every strictly-lower block is also written
  // transposed, which fills the rest.  blk(x) = x / 16 (bf16) or x / 32.
  constexpr int kBlkShift = (DT == kBF16) ? 4 : 5;
  auto upper = [&](int row, int col) { return diag && (col >> kBlkShift) > (row >> kBlkShift); };
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    if (wr == h) stage_acc(lds, acc, alpha);
    __syncthreads();
    if (square) {
      // B = cq A A + cl A: add cl times this half-tile of A (its own rows; A
      // is symmetric, so the mirrored copy below stays consistent)
#pragma unroll 4
      for (int k = 0; k < (128 * 64 / kThreads); ++k) {
        const int r = (tid >> 6) + (kThreads / 64) * k, c = tid & 63;
        if (upper(128 * h + r, 4 * c)) continue;
        float av[4];
        vld4(a_in + static_cast<long>(Rt + 128 * h + r) * mp + Ct + 4 * c, av);
        const float4 v4 = stage_ld4(lds, r, c);
        stage_st4(lds, r, c, make_float4(fmaf(cl, av[0], v4.x), fmaf(cl, av[1], v4.y), fmaf(cl, av[2], v4.z),
                                         fmaf(cl, av[3], v4.w)));
      }
      __syncthreads();
    }
    // A rows: thread covers chunk tid & 63 of rows (tid >> 6) + 8 k
#pragma unroll 4
    for (int k = 0; k < (128 * 64 / kThreads); ++k) {
      const int r = (tid >> 6) + (kThreads / 64) * k, c = tid & 63;
      if (upper(128 * h + r, 4 * c)) continue;
      const float4 v4 = stage_ld4(lds, r, c);
      const float v[4] = {v4.x, v4.y, v4.z, v4.w};
      vst4(a + static_cast<long>(Rt + 128 * h + r) * mp + Ct + 4 * c, v);
    }
    if (mirror || diag) {
      // transposed copy into the upper triangle: 8-row segments of columns
      // (of a diagonal tile only the strictly-lower blocks)
#pragma unroll 2
      for (int j = 0; j < 256 * 16 / kThreads; ++j) {
        const int q = tid + kThreads * j, sgi = q & 15, col = q >> 4;
        if (diag && !upper(col, 128 * h + 8 * sgi)) continue;
        float v[8];
        stage_col8(lds, sgi, col, v);
        vst8(a + static_cast<long>(Ct + col) * mp + Rt + 128 * h + 8 * sgi, v);
      }
    }
    __syncthreads();
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads, 1) void ns_gemm_kernel(const MatDesc* __restrict__ descs, SegTable st,
                                                             const MatScale* __restrict__ scales, int step,
                                                             int last, int mode, float lr, float decay,
                                                             float cx, float cax, int poly) {
  using T = typename Elem<DT>::T;
  constexpr int EB = Elem<DT>::kBytes;
  __shared__ __attribute__((aligned(16))) char lds[2 * kStageBytes];

  const TileRef tr = locate(st, blockIdx.x, false);
  const MatDesc& d = descs[tr.mat];
  const int mp = d.mp, np = d.np;
  const char* a = static_cast<const char*>(poly ? d.b : d.a);
  // X of this step (operand copy) and the copy the epilogue writes for the next
  const char* xq = static_cast<const char*>((step & 1) ? d.xs1 : d.xs0);
  T* xs_next = static_cast<T*>((step & 1) ? d.xs0 : d.xs1);
  const long lda = static_cast<long>(mp) * EB;

  Acc<DT> acc;
  zero_acc<DT>(acc);

  const float gamma = (step == 0) ? scales[tr.mat].c : 1.0f;
  const int tid = threadIdx.x, wr = (tid >> 6) / Grid::kWN;
  const int Rt = tr.bi * kTile, Ct = tr.bj * kTile;
  // The iterate: fp32 moves from xq to xs_next; bf16 is the pair hi (xq, then
  // xs_next) + lo (xm, in place)
  const float* xold = reinterpret_cast<const float*>(xq);
  float* xnew = reinterpret_cast<float*>(xs_next);
  __bf16* xlo = static_cast<__bf16*>(d.xm);
  const bool trn = d.tr != 0;
  const float step_lr = -lr * d.lr_scale;
  // The tile is finished in four 64-row quarters through two 64 KB LDS
  // buffers.  Quarter q is tile rows 32 q .. 32 q + 31 and 128 + 32 q ..
  // 128 + 32 q + 31, i.e. accumulator block mi = q of every wave, so all
  // eight waves share each quarter's work.  Its iterate rows arrive by
  // LDS-DMA (fp32: 16-byte chunk c of a row holds columns 4c..4c+3; bf16:
  // chunk 2c holds hi and chunk 2c + 1 lo of columns 8c..8c+7); each wave
  // replaces its part by gamma (cx X + cax A X) in fp32 (for bf16 the two
  // lanes sharing a chunk pair read it in the same instructions, then write
  // their fp32 columns over it); then every wave reads its rows into
  // registers, the buffer is handed to quarter q + 2's DMA, and the rows are
  // stored.  vmcnt counts loads and stores in issue order, so each wait for a
  // quarter's DMA leaves the stores issued after it in flight.
  constexpr int kQRows = 64;
  constexpr int kQBytes = kQRows * 1024;
  constexpr int kDmaRows = kQRows / (kThreads / 64);         // rows per wave per quarter
  constexpr int kRowIt = kQRows * 64 / kThreads;             // row chunks per thread per quarter
  constexpr int kColIt = 256 * (kQRows / 8) / kThreads;      // column segments per thread per quarter
  // store instructions per thread per quarter on a non-final step
  constexpr int kStoresQ = (DT == kBF16) ? 2 * kRowIt : kRowIt;
  static_assert(2 * kStoresQ + kDmaRows < 64, "vmcnt range");
  const int c = tid & 63, col = Ct + 4 * c;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int cbase = (wave % Grid::kWN) * kBN * 8;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(lds));
  // tile row of row i (0..63) of quarter q's buffer
  auto qrow = [](int q, int i) { return (i < 32) ? 32 * q + i : 96 + 32 * q + i; };
  const char* xtile = uniform_ptr(reinterpret_cast<const char*>(xold + static_cast<long>(Rt) * np + Ct));
  const char* hi_tile = xq + (static_cast<long>(Rt) * np + Ct) * 2;
  const char* lo_tile = reinterpret_cast<const char*>(xlo + static_cast<long>(Rt) * np + Ct);
  // row i (0 .. kDmaRows - 1) of this wave's share of quarter q's DMA
  auto dma_quarter_row = [&](int q, int i) {
    const uint32_t dst = lds0 + (q & 1) * kQBytes;
    const int r = wave * kDmaRows + i;
    const int ls = lane ^ ((r ^ (r >> 3)) & 63);   // logical chunk of this lane's slot
    if constexpr (DT == kBF16) {
      const char* src = ((ls & 1) ? lo_tile : hi_tile) + static_cast<long>(qrow(q, r)) * np * 2 + (ls >> 1) * 16;
      lds_dma16_addr_nt(src, dst + r * 1024);
    } else {
      lds_dma16(xtile, static_cast<uint32_t>(qrow(q, r) * np * 4 + 16 * ls), dst + r * 1024);
    }
  };
  auto dma_quarter = [&](int q) {
#pragma unroll
    for (int i = 0; i < kDmaRows; ++i) dma_quarter_row(q, i);
  };
  // quarter 0 lands in the buffer the second-to-last stage frees, a stage
  // before the product ends; quarter 1 starts at the last barrier
  static_assert(kDmaRows == 2 * Grid::kLoadsPerOperand, "one early load per main-loop DMA slot");
  if constexpr (DT == kBF16)
    block_product16<true>(a + static_cast<long>(tr.bi) * kTile * lda, lda, xq + static_cast<long>(tr.bj) * kTile * EB,
                          np * EB, mp * EB, lds, acc, [&](int i) { dma_quarter_row(0, i); }, [&] { dma_quarter(1); });
  else
    block_product<DT, kWaves, true>(a + static_cast<long>(tr.bi) * kTile * lda, lda,
                                    xq + static_cast<long>(tr.bj) * kTile * EB, np * EB, mp * EB, lds, acc,
                                    [&](int i) { dma_quarter_row(0, i); }, [&] { dma_quarter(1); });
  wait_vmcnt<kDmaRows>();
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    char* buf = lds + (q & 1) * kQBytes;
    if constexpr (DT == kBF16) {
      // quarter q is 16 x 16 blocks mi = 2 q + m2 of every wave: lane l holds
      // buffer row 32 wr + 16 m2 + (l & 15), columns 4 c4 .. 4 c4 + 3 with
      // c4 = cbase + 4 ni + (l >> 4), i.e. half (l >> 4) & 1 of chunk pair
      // (c4 & ~1, c4 | 1).  All reads of the block first, then the updates.
      const int l16 = lane & 15, lq = lane >> 4;
      float4 xv[2][4];
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int r = 32 * wr + 16 * m2 + l16, c4 = cbase + 4 * ni + lq;
          const bf16x4 h = *reinterpret_cast<const bf16x4*>(buf + stage_off(r, c4 & ~1) + 8 * (lq & 1));
          const bf16x4 l = *reinterpret_cast<const bf16x4*>(buf + stage_off(r, c4 | 1) + 8 * (lq & 1));
          xv[m2][ni] = make_float4(static_cast<float>(h[0]) + static_cast<float>(l[0]),
                                   static_cast<float>(h[1]) + static_cast<float>(l[1]),
                                   static_cast<float>(h[2]) + static_cast<float>(l[2]),
                                   static_cast<float>(h[3]) + static_cast<float>(l[3]));
        }
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const float4 x = xv[m2][ni];
          const f32x4& ax = acc[2 * q + m2][ni];
          *reinterpret_cast<float4*>(buf + stage_off(32 * wr + 16 * m2 + l16, cbase + 4 * ni + lq)) =
              make_float4(gamma * (cx * x.x + cax * ax[0]), gamma * (cx * x.y + cax * ax[1]),
                          gamma * (cx * x.z + cax * ax[2]), gamma * (cx * x.w + cax * ax[3]));
        }
    } else {
      // all reads of the block first, then the updates (one LDS round trip)
      float4 xv[kBN][4];
#pragma unroll
      for (int ni = 0; ni < kBN; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          xv[ni][g] = *reinterpret_cast<const float4*>(buf + stage_off(32 * wr + li, cbase + 8 * ni + 2 * g + lh));
#pragma unroll
      for (int ni = 0; ni < kBN; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 x = xv[ni][g];
          const f32x16& ax = acc[q][ni];
          *reinterpret_cast<float4*>(buf + stage_off(32 * wr + li, cbase + 8 * ni + 2 * g + lh)) =
              make_float4(gamma * (cx * x.x + cax * ax[4 * g]), gamma * (cx * x.y + cax * ax[4 * g + 1]),
                          gamma * (cx * x.z + cax * ax[4 * g + 2]), gamma * (cx * x.w + cax * ax[4 * g + 3]));
        }
    }
    __syncthreads();
    if (!last) {
      // iterate rows: fp32, or the bf16 pair (hi is the next step's operand copy)
      f32v4 rv[kRowIt];
#pragma unroll
      for (int k = 0; k < kRowIt; ++k) {
        const float4 v4 = stage_ld4(buf, (tid >> 6) + (kThreads / 64) * k, c);
        rv[k] = f32v4{v4.x, v4.y, v4.z, v4.w};
      }
      if (q < 2) {
        __syncthreads();         // every wave holds its rows: the buffer is free
        dma_quarter(q + 2);
      }
#pragma unroll
      for (int k = 0; k < kRowIt; ++k) {
        const int row = Rt + qrow(q, (tid >> 6) + (kThreads / 64) * k);
        const float xn[4] = {rv[k].x, rv[k].y, rv[k].z, rv[k].w};
        if constexpr (DT == kBF16) {
          float hi[4], lo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hi[e] = static_cast<float>(static_cast<__bf16>(xn[e]));
            lo[e] = xn[e] - hi[e];
          }
          vst4_nt(xs_next + static_cast<long>(row) * np + col, hi);
          vst4_nt(xlo + static_cast<long>(row) * np + col, lo);
        } else {
          vst4(xnew + static_cast<long>(row) * np + col, xn);
        }
      }
      // wait for quarter q + 1's DMA; what was issued after it stays in flight
      if (q == 0) wait_vmcnt<kDmaRows + kStoresQ>();
      else if (q == 1) wait_vmcnt<2 * kStoresQ + kDmaRows>();
      else if (q == 2) wait_vmcnt<2 * kStoresQ>();
      if (q < 3) __syncthreads();
    } else {
      if (!trn) {
        // final step, wide matrix: caller rows
#pragma unroll
        for (int k = 0; k < kRowIt; ++k) {
          const int r = (tid >> 6) + (kThreads / 64) * k;
          const float4 v4 = stage_ld4(buf, r, c);
          const float xn[4] = {v4.x, v4.y, v4.z, v4.w};
          write_caller<T, 4>(d, mode, step_lr, decay, Rt + qrow(q, r), col, xn);
        }
      } else {
        // final step, tall matrix: wide (row, col) is caller (col, row); an
        // 8-row segment never straddles the quarter's two 32-row blocks
#pragma unroll
        for (int j = 0; j < kColIt; ++j) {
          const int qq = tid + kThreads * j, sgi = qq & 7, col8 = qq >> 3;
          float v[8];
          stage_col8(buf, sgi, col8, v);
          write_caller<T, 8>(d, mode, step_lr, decay, Ct + col8, Rt + qrow(q, 8 * sgi), v);
        }
      }
      if (q < 3) {
        wait_vmcnt<0>();
        __syncthreads();
        if (q < 2) dma_quarter(q + 2);  // into the buffer quarter q just released
      }
    }
  }
}


// ---------------------------------------------------------------- small fp32 tiles
// fp32 matrices of at most two 256-tile rows (m' <= 512) give too few 256 x 256
// tiles to occupy 256 CUs: the TinyMLP set's update is 192 of them, its Gram
// 36.  The two kernels below compute the same products on 128 x 128 tiles (4x
// the blocks): four waves in a 2 x 2 grid of 64 x 64 blocks, each 2 x 2
// v_mfma_f32_32x32x2_f32 blocks.  An fp32 MFMA occupies its SIMD for 64 cycles,
// so register-staged loads into padded LDS rows keep it fed.  The epilogues
// work straight from the accumulators (lane (li, lh), register 4 g + q of
// block (mi, ni) is C[64 wr + 32 mi + li][64 wc + 32 ni + 8 g + 4 lh + q], as
// above).
constexpr int kSmThreads = 256;
// K per stage: two stages of 16 take 40 KB of LDS and at most 128 VGPRs, so
// four workgroups share a CU and the TinyMLP set's 768 update tiles are all
// resident at once (stages of 32 with two workgroups per CU: update launch
// 0.131 against 0.125 ms, the Gram 0.045 against 0.047 ms, the step the same
// to 1%)
constexpr int kSmK = 16;
constexpr int kSmWg = 4;                // workgroups per CU
constexpr int kSmRowFloats = kSmK + 4;  // K-contiguous LDS row: + 4 floats (16-byte reads of 16 rows: distinct banks)
constexpr int kSmCpr = kSmK / 4;        // 16-byte chunks per K-contiguous stage row
constexpr int kSmLd = kSmK / 8;         // 16-byte loads per thread per operand and stage
constexpr int kSmQnRowFloats = 136;     // row-major stage row: 128 floats + 8 (rows 4 apart land 32 banks apart)
constexpr int kSmPFloats = kSmallTile * kSmRowFloats;
constexpr int kSmStageFloats = 2 * kSmPFloats;   // P + Q (a row-major Q stage needs only kSmK * kSmQnRowFloats)
static_assert(kSmK * kSmQnRowFloats <= kSmPFloats, "row-major stage fits the Q region");

// acc[mi][ni] of wave (wr, wc) += its 64 x 64 block (rows 64 wr.., cols
// 64 wc..) of P Q^T over K = klen, a multiple of kSmK.  P: 128 rows,
// K-contiguous, pitch ldp floats.  Q: QN == false like P (its rows are output
// columns); QN == true K rows of the 128 output columns, pitch ldq.  In each
// stage, K index 8 u + 4 h + e is element e of the float4 that the lanes of
// half h read for group u, for both operands alike, so every k is summed once.
// kMask: bit 2 mi + ni set when block (mi, ni) is needed (the others' MFMAs and
// unused fragment reads are skipped; the wave still loads and joins barriers).
template <bool QN, unsigned kMask = 0xFu>
__device__ __forceinline__ void small_product(const float* __restrict__ P, long ldp, const float* __restrict__ Q,
                                              long ldq, int klen, float* lds, f32x16 (&acc)[2][2]) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1, li = lane & 31, lh = lane >> 5;
  // K-contiguous operands: thread t loads chunk t % kSmCpr of rows
  // t / kSmCpr + (256 / kSmCpr) j; a row-major Q: 16 bytes at column 4 (t & 31)
  // of K rows (t >> 5) + 8 j
  f32v4 rp[kSmLd], rq[kSmLd];
  const int crow = t / kSmCpr, cch = 4 * (t % kSmCpr);
  constexpr int kRowStep = kSmThreads / kSmCpr;
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < kSmLd; ++j) {
      rp[j] = *gmem(reinterpret_cast<const f32v4*>(P + static_cast<long>(crow + kRowStep * j) * ldp + k0 + cch));
      if constexpr (QN)
        rq[j] = *gmem(reinterpret_cast<const f32v4*>(Q + static_cast<long>(k0 + (t >> 5) + 8 * j) * ldq + 4 * (t & 31)));
      else
        rq[j] = *gmem(reinterpret_cast<const f32v4*>(Q + static_cast<long>(crow + kRowStep * j) * ldq + k0 + cch));
    }
  };
  auto store = [&](float* st) {
#pragma unroll
    for (int j = 0; j < kSmLd; ++j) {
      *reinterpret_cast<f32v4*>(st + (crow + kRowStep * j) * kSmRowFloats + cch) = rp[j];
      if constexpr (QN)
        *reinterpret_cast<f32v4*>(st + kSmPFloats + ((t >> 5) + 8 * j) * kSmQnRowFloats + 4 * (t & 31)) = rq[j];
      else
        *reinterpret_cast<f32v4*>(st + kSmPFloats + (crow + kRowStep * j) * kSmRowFloats + cch) = rq[j];
    }
  };
  auto compute = [&](const float* st) {
#pragma unroll
    for (int u = 0; u < kSmK / 8; ++u) {
      f32v4 fa[2] = {}, fb[2] = {};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if ((kMask >> (2 * i)) & 3u)
          fa[i] = *reinterpret_cast<const f32v4*>(st + (64 * wr + 32 * i + li) * kSmRowFloats + 8 * u + 4 * lh);
        if (((kMask >> i) & 5u) == 0u) continue;
        if constexpr (QN) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            fb[i][e] = st[kSmPFloats + (8 * u + 4 * lh + e) * kSmQnRowFloats + 64 * wc + 32 * i + li];
        } else {
          fb[i] = *reinterpret_cast<const f32v4*>(st + kSmPFloats + (64 * wc + 32 * i + li) * kSmRowFloats + 8 * u +
                                                  4 * lh);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            if ((kMask >> (2 * mi + ni)) & 1u)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[ni][e], fa[mi][e], acc[mi][ni], 0, 0, 0);
    }
  };
  // two stages: stage s + 1's loads are in flight while stage s is multiplied
  const int ns = klen / kSmK;
  load(0);
  store(lds);
  __syncthreads();
  for (int s = 0; s < ns; ++s) {
    if (s + 1 < ns) load((s + 1) * kSmK);
    compute(lds + (s & 1) * kSmStageFloats);
    if (s + 1 < ns) store(lds + ((s + 1) & 1) * kSmStageFloats);
    __syncthreads();
  }
}

// A split small tile's partial product, by thread as for the 256 tiles.
__device__ __forceinline__ void small_store_partial(float* part, const f32x16 (&acc)[2][2]) {
  f32v4* dst = reinterpret_cast<f32v4*>(part) + threadIdx.x;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x16& a = acc[b >> 1][b & 1];
      *gmem(dst + (b * 4 + g) * kSmThreads) = f32v4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
    }
}

__device__ __forceinline__ void small_add_partial(const float* part, f32x16 (&acc)[2][2]) {
  const f32v4* src = reinterpret_cast<const f32v4*>(part) + threadIdx.x;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32v4 v = *gmem(src + (b * 4 + g) * kSmThreads);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[b >> 1][b & 1][4 * g + e] += v[e];
    }
}

// One caller element of the last step (the transposed write of a tall matrix):
// the same arithmetic as write_caller.
__device__ __forceinline__ void write_caller1(const MatDesc& d, int mode, float step_lr, float decay, int orow,
                                              int ocol, float u) {
  if (orow >= d.m || ocol >= d.n) return;
  const long o = static_cast<long>(orow) * d.n + ocol;
  float* p = static_cast<float*>(d.p);
  if (mode == kModeMuon) {
    gmem(p)[o] = fmaf(step_lr, u, gmem(p)[o] * decay);
    if (d.upd) gmem(d.upd)[o] = u;
  } else {
    gmem(p)[o] = u;
  }
}

// The Gram product on 128 x 128 tiles (fp32): as syrk_kernel.  A diagonal
// tile computes only its 32 x 32 blocks on or below the block diagonal and
// writes the strictly-lower ones transposed as well.
__global__ __launch_bounds__(kSmThreads, kSmWg) void small_syrk_kernel(const MatDesc* __restrict__ descs, SegTable st,
                                                                   const MatScale* __restrict__ scales, int step,
                                                                   int square, float cq, float cl, int reduce) {
  __shared__ __attribute__((aligned(16))) float lds[2 * kSmStageFloats];
  const TileRef tr = locate(st, blockIdx.x, true, reduce != 0, kSmallPartialFloats);
  const MatDesc& d = descs[tr.mat];
  const int mp = d.mp;
  const float* xs = static_cast<const float*>(square ? d.a : ((step & 1) ? d.xs1 : d.xs0));
  const int kdim = square ? mp : d.np;

  f32x16 acc[2][2];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b >> 1][b & 1] = f32x16{};
  const bool diag = tr.bi == tr.bj && !tr.full;
  if (!reduce) {
    const int klen = kdim / tr.ksplit;
    const long koff = static_cast<long>(tr.slice) * klen;
    const float* p = xs + static_cast<long>(tr.bi) * kSmallTile * kdim + koff;
    const float* q = xs + static_cast<long>(tr.bj) * kSmallTile * kdim + koff;
    // block (R, C) = (2 wr + mi, 2 wc + ni) of a diagonal tile is needed when C <= R
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int band = (wv & 1) - (wv >> 1);
    auto run = [&](auto mask) {
      small_product<false, decltype(mask)::value>(p, kdim, q, kdim, klen, lds, acc);
    };
    if (!diag || band < 0) run(std::integral_constant<unsigned, 0xFu>{});
    else if (band == 0) run(std::integral_constant<unsigned, 0xDu>{});     // all but block (0, 1)
    else run(std::integral_constant<unsigned, 0x0u>{});
    if (tr.ksplit > 1) {
      small_store_partial(tr.part + static_cast<long>(tr.slice) * kSmallPartialFloats, acc);
      return;
    }
  } else {
    for (int s = 0; s < tr.ksplit; ++s) small_add_partial(tr.part + static_cast<long>(s) * kSmallPartialFloats, acc);
  }

  const float alpha = square ? cq : (step == 0 ? scales[tr.mat].c2 : 1.0f);
  float* out = static_cast<float*>(square ? d.b : d.a);
  const float* a_in = static_cast<const float*>(d.a);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1, li = lane & 31, lh = lane >> 5;
  const bool mirror = tr.bi != tr.bj && !tr.full;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = tr.bi * kSmallTile + 64 * wr + 32 * mi + li;
        const int c = tr.bj * kSmallTile + 64 * wc + 32 * ni + 8 * g + 4 * lh;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[mi][ni][4 * g + q] * alpha;
        if (square) {
          // B = cq A A + cl A
          float av[4];
          vld4(a_in + static_cast<long>(r) * mp + c, av);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = fmaf(cl, av[q], v[q]);
        }
        // diagonal tile: blocks above the block diagonal are not computed,
        // those below it are also written transposed
        const int br = (r - tr.bi * kSmallTile) >> 5, bc = (c - tr.bj * kSmallTile) >> 5;
        if (diag && bc > br) continue;
        vst4(out + static_cast<long>(r) * mp + c, v);
        if (mirror || (diag && br > bc)) {
#pragma unroll
          for (int q = 0; q < 4; ++q) gmem(out)[static_cast<long>(c + q) * mp + r] = v[q];
        }
      }
}

// The update on 128 x 128 tiles (fp32): as ns_gemm_kernel.
__global__ __launch_bounds__(kSmThreads, kSmWg) void small_gemm_kernel(const MatDesc* __restrict__ descs, SegTable st,
                                                                   const MatScale* __restrict__ scales, int step,
                                                                   int last, int mode, float lr, float decay,
                                                                   float cx, float cax, int poly) {
  __shared__ __attribute__((aligned(16))) float lds[2 * kSmStageFloats];
  const TileRef tr = locate(st, blockIdx.x, false);
  const MatDesc& d = descs[tr.mat];
  const int mp = d.mp, np = d.np;
  const float* m = static_cast<const float*>(poly ? d.b : d.a);
  // the iterate: read from this step's buffer, written to the other one
  const float* xq = static_cast<const float*>((step & 1) ? d.xs1 : d.xs0);
  float* xnext = static_cast<float*>((step & 1) ? d.xs0 : d.xs1);

  f32x16 acc[2][2];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b >> 1][b & 1] = f32x16{};
  small_product<true>(m + static_cast<long>(tr.bi) * kSmallTile * mp, mp, xq + static_cast<long>(tr.bj) * kSmallTile,
                      np, mp, lds, acc);

  const float gamma = (step == 0) ? scales[tr.mat].c : 1.0f;
  const float step_lr = -lr * d.lr_scale;
  const bool trn = d.tr != 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1, li = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = tr.bi * kSmallTile + 64 * wr + 32 * mi + li;
        const int c = tr.bj * kSmallTile + 64 * wc + 32 * ni + 8 * g + 4 * lh;
        float x[4], xn[4];
        vld4(xq + static_cast<long>(r) * np + c, x);
#pragma unroll
        for (int q = 0; q < 4; ++q) xn[q] = gamma * (cx * x[q] + cax * acc[mi][ni][4 * g + q]);
        if (!last) {
          vst4(xnext + static_cast<long>(r) * np + c, xn);
        } else if (!trn) {
          write_caller<float, 4>(d, mode, step_lr, decay, r, c, xn);
        } else {
          // tall: wide (r, c + q) is caller (c + q, r)
#pragma unroll
          for (int q = 0; q < 4; ++q) write_caller1(d, mode, step_lr, decay, c + q, r, xn[q]);
        }
      }
}

}  // namespace

hipError_t launch_syrk(int dt, const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales,
                       int step, int square, float cq, float cl, int reduce, hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(syrk_kernel<kBF16>, dim3(ntiles), dim3(kThreads), 0, stream, descs, st, scales, step,
                       square, cq, cl, reduce);
  else
    hipLaunchKernelGGL(syrk_kernel<kF32>, dim3(ntiles), dim3(kThreads), 0, stream, descs, st, scales, step,
                       square, cq, cl, reduce);
  return hipGetLastError();
}

hipError_t launch_ns_gemm(int dt, const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales,
                          int step, int last, int mode, float lr, float decay, float cx, float cax, int poly,
                          hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(ns_gemm_kernel<kBF16>, dim3(ntiles), dim3(kThreads), 0, stream, descs, st, scales, step, last,
                       mode, lr, decay, cx, cax, poly);
  else
    hipLaunchKernelGGL(ns_gemm_kernel<kF32>, dim3(ntiles), dim3(kThreads), 0, stream, descs, st, scales, step, last,
                       mode, lr, decay, cx, cax, poly);
  return hipGetLastError();
}

hipError_t launch_small_syrk(const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales, int step,
                             int square, float cq, float cl, int reduce, hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(small_syrk_kernel, dim3(ntiles), dim3(kSmThreads), 0, stream, descs, st, scales, step, square,
                     cq, cl, reduce);
  return hipGetLastError();
}

hipError_t launch_small_gemm(const MatDesc* descs, const SegTable& st, int ntiles, const MatScale* scales, int step,
                             int last, int mode, float lr, float decay, float cx, float cax, int poly,
                             hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(small_gemm_kernel, dim3(ntiles), dim3(kSmThreads), 0, stream, descs, st, scales, step, last, mode,
                     lr, decay, cx, cax, poly);
  return hipGetLastError();
}

}  // namespace dmuon
