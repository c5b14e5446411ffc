// Helpers shared by the MFMA (gfx950 matrix core) kernels.
//
// Operand layout of v_mfma_f32_32x32x16_bf16 as used here (one wave64):
//   A (32 x 16): lane l holds row l%32, eight k-slots of half l/32;
//   B (16 x 32): lane l holds column l%32, the same eight k-slots;
//   C (32 x 32): lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4
//                in its 16 accumulator registers i = 0..15.
// The kernels rely only on A and B numbering their k-slots the same way,
// so a C tile can be fed back as a B operand after a fixed permutation of
// the contraction index (see perm16 below).
#pragma once

#include "common.h"

namespace dualkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Exchange a value with the lane 32 positions away (the other half of the
// wave): C-tile rows held by the two halves are disjoint.  v_permlane32_swap
// swaps the upper half of its first operand with the lower half of its
// second, so with both set to x each lane finds its partner's value in the
// result that its own half did not keep.
__device__ __forceinline__ float swap_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// A C tile of 32 keys feeds the B operand of the next product in two
// 16-key steps.  Register i of half h holds key 8*(i/4) + 4*h + i%4, so
// step s (registers 8s .. 8s+7) holds, in k-slot j of half h, key
// 16*s + w with w = 8*(j/4) + 4*h + j%4.  Storing the other operand with
// key w at position 8*h + j -- i.e. bits 2 and 3 of w swapped -- lines
// both operands up.
__device__ __forceinline__ int perm16(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Workgroup -> logical block.  A launch's work is `units` groups of
// `per_unit` logical blocks (a head group with its query blocks, or a KV
// head with its key items), each group in longest-first order.  Workgroups
// are dispatched round robin over the 8 XCDs (workgroup b runs on XCD b % 8
// as that XCD's (b / 8)-th), and each XCD has its own L2.  So that every XCD
// works on one unit's data at a time AND gets the same share of the work:
//  * units a multiple of 8: XCD x takes whole units x, x + 8, ...;
//  * 8 a multiple of units: S = 8 / units XCDs share a unit, XCD x taking
//    every S-th block of it (offset x % S); the grid is padded to whole
//    rounds and padding workgroups get -1;
//  * otherwise the natural order.
__device__ __forceinline__ int balanced_block(int bid, int units, int per_unit) {
  constexpr int X = 8;
  const int xcd = bid % X, slot = bid / X;
  if (units % X == 0) {
    const int k = slot / per_unit, item = slot - k * per_unit;
    return (xcd + X * k) * per_unit + item;
  }
  if (X % units == 0) {
    const int S = X / units;
    const int item = slot * S + xcd % S;
    return item < per_unit ? (xcd / S) * per_unit + item : -1;
  }
  return bid;
}

// GEMM tile of workgroup `bid` on a tm x tn grid of C tiles.  The grid is
// cut into blocks of 4 x 8 (or 8 x 4) tiles, numbered row by row; XCD x
// (the workgroups bid = x mod 8) walks the x-th eighth of that numbering,
// so the 32 workgroups it runs at a time (one per CU) are one block and
// its L2 sees 12 distinct operand panels per k-step instead of the 18 of a
// row-major walk.  Grids that do not split into such blocks stay row-major.
__device__ __forceinline__ void gemm_tile_of(int bid, int tm, int tn, int& bm, int& bn) {
  constexpr int X = 8, PER = 32;
  const int sn = tn % 8 == 0 ? 8 : 4, sm = PER / sn;
  if (tn % sn != 0 || tm % sm != 0) {
    bm = bid / tn;
    bn = bid % tn;
    return;
  }
  const int q = (bid % X) * (tm * tn / X) + bid / X;   // position in block order
  const int blk = q / PER, in = q % PER;
  const int bpr = tn / sn;                             // blocks per block row
  bm = (blk / bpr) * sm + in / sn;
  bn = (blk % bpr) * sn + in % sn;
}

// Grid size for balanced_block.
inline int64_t balanced_grid(int units, int64_t per_unit) {
  constexpr int X = 8;
  if (units % X != 0 && X % units == 0) {
    const int S = X / units;
    return X * ((per_unit + S - 1) / S);
  }
  return (int64_t)units * per_unit;
}

// Query heads handled together by one workgroup: the largest power of two
// that divides the GQA group size and is at most `waves`.
inline int heads_per_block(int g, int waves) {
  int hg = 1;
  while (hg * 2 <= waves && g % (hg * 2) == 0) hg *= 2;
  return hg;
}

// Query row blocks of the packed layout, longest key range first:
// response blocks (their keys span the whole prompt) by decreasing row
// index within the response, then prompt blocks by decreasing row.
struct RowBlock {
  int seg;       // -1 prompt, else response index n
  int r0;        // first row of the block inside its segment
  int base;      // packed row of the segment's row 0
  int seglen;    // P or R: rows r < seglen belong to the segment
  int nvalid;    // P or the valid length of response n
  int posoff;    // logical position of the segment's row 0 (0 or P)
};

__device__ __forceinline__ RowBlock decode_block(const Problem& pr, int blk, int BM, int nbP,
                                                 int nbR) {
  RowBlock b;
  if (blk < pr.N * nbR) {
    const int rb = nbR - 1 - blk / pr.N;
    b.seg = blk % pr.N;
    b.r0 = rb * BM;
    b.base = pr.P + b.seg * pr.R;
    b.seglen = pr.R;
    b.nvalid = resp_valid(pr, b.seg);
    b.posoff = pr.P;
  } else {
    const int pb = nbP - 1 - (blk - pr.N * nbR);
    b.seg = -1;
    b.r0 = pb * BM;
    b.base = 0;
    b.seglen = pr.P;
    b.nvalid = pr.P;
    b.posoff = 0;
  }
  return b;
}

// Key tiles of BN rows visited by a query block whose valid rows are
// [r_lo, r_hi] of segment `b`: tiles [a0, a0+nA) of the prompt (phase A),
// then tiles [b0, b0+nB) of the block's own response (phase B).  For a
// prompt block phase A is the causal range and phase B is empty.
struct TileRange {
  int a0, nA, b0, nB;
};

__device__ __forceinline__ TileRange key_tiles(const Problem& pr, const RowBlock& b, int r_lo,
                                               int r_hi, int BN) {
  TileRange t{0, 0, 0, 0};
  const int q_lo = b.posoff + r_lo, q_hi = b.posoff + r_hi;
  const int kp_lo = pr.W > 0 ? max(0, q_lo - pr.W + 1) : 0;   // lowest visible position
  if (b.seg < 0) {
    t.a0 = kp_lo / BN;
    t.nA = q_hi / BN + 1 - t.a0;
    return t;
  }
  if (kp_lo < pr.P) {
    t.a0 = kp_lo / BN;
    t.nA = (pr.P + BN - 1) / BN - t.a0;
  }
  t.b0 = max(0, kp_lo - pr.P) / BN;
  t.nB = r_hi / BN + 1 - t.b0;
  return t;
}

// Per-tile key description: packed row of key 0, its logical position, and
// how many of the BN keys are real (keys >= lim are masked and zero-filled).
struct KeyTile {
  int row0, pos0, lim;
};

__device__ __forceinline__ KeyTile tile_at(const Problem& pr, const RowBlock& b,
                                           const TileRange& t, int it, int BN) {
  KeyTile k;
  if (it < t.nA) {
    const int kt = t.a0 + it;
    k.row0 = kt * BN;
    k.pos0 = kt * BN;
    k.lim = pr.P - kt * BN;
  } else {
    const int kt = t.b0 + (it - t.nA);
    k.row0 = b.base + kt * BN;
    k.pos0 = pr.P + kt * BN;
    k.lim = b.nvalid - kt * BN;
  }
  return k;
}

// How a wave whose valid query positions are [qlo, qhi] (all of its 32 rows
// valid iff `all_valid`) treats a key tile: 0 skip, 1 full, 2 masked.
__device__ __forceinline__ int tile_kind(const Problem& pr, const KeyTile& kt, int BN, bool any_valid,
                                         bool all_valid, int qlo, int qhi) {
  if (!any_valid || kt.lim <= 0 || kt.pos0 > qhi) return 0;
  const int kmax = kt.pos0 + min(BN, kt.lim) - 1;
  if (pr.W > 0 && qlo - kmax >= pr.W) return 0;
  const bool full = all_valid && kt.lim >= BN && kt.pos0 + BN - 1 <= qlo &&
                    (pr.W <= 0 || qhi - kt.pos0 < pr.W);
  return full ? 1 : 2;
}

// Set a pair of LDS/HIP launch attributes once per kernel instantiation.
template <typename F>
inline hipError_t allow_lds(F* kern, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

}  // namespace dualkv
