// Global -> LDS staging of bf16 row tiles for the MFMA kernels.
//
// A tile is ROWS consecutive packed rows of one head (D bf16 each).  Every
// thread loads pairs of rows x 8 head dims with two 128-bit loads (16
// lanes cover one 256-byte row segment, so loads coalesce), then writes
//  * row-major:  dst[row * STRIDE + dim]   (STRIDE = D + 8: the 16-byte pad
//                makes the 128-bit operand reads of 8 consecutive rows hit
//                distinct banks), and/or
//  * transposed: dst[dim * ROWS + phys(row)] where rows are placed in the
//                perm16 order that matches a C tile re-used as a B operand,
//                and 16-byte chunks are XOR-swizzled per dim row.
// Rows >= nrows are zero-filled, so masked rows never inject NaN/Inf.
#pragma once

#include "mfma_common.h"

namespace dualkv {

template <int ROWS>
__device__ __forceinline__ int trans_swz(int d) {
  return ((d & 7) ^ ((d >> 3) & 7)) & (ROWS / 8 - 1);
}

// Position of (dim d, row r) in a transposed tile.
template <int ROWS>
__device__ __forceinline__ int trans_index(int d, int r) {
  const int pos = perm16(r);
  return d * ROWS + ((((pos >> 3) ^ trans_swz<ROWS>(d)) << 3) | (pos & 7));
}

// 128-bit operand read of a transposed tile: dim row d, k-step `ks` (16
// rows), wave half `hf`.
template <int ROWS>
__device__ __forceinline__ bf16x8 trans_read(const uint16_t* t, int d, int ks, int hf) {
  return *reinterpret_cast<const bf16x8*>(t + d * ROWS + (((2 * ks + hf) ^ trans_swz<ROWS>(d)) << 3));
}

template <int ROWS, int D, int NT>
struct PairTile {
  static constexpr int STRIDE = D + 8;
  static constexpr int G = (ROWS / 2) * (D / 8);
  static constexpr int PT = (G + NT - 1) / NT;
  uint4 r[PT][2];

  // rows [0, nrows) of the tile whose row 0 is at `base`, row stride `rs`
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t rs, int nrows,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int gi = tid + i * NT;
      const int c8 = gi % (D / 8), rp = gi / (D / 8);
      uint4 z0 = {0, 0, 0, 0}, z1 = {0, 0, 0, 0};
      if (G % NT == 0 || gi < G) {
        const uint16_t* p = base + (int64_t)(2 * rp) * rs + c8 * 8;
        if (2 * rp < nrows) z0 = *reinterpret_cast<const uint4*>(p);
        if (2 * rp + 1 < nrows) z1 = *reinterpret_cast<const uint4*>(p + rs);
      }
      r[i][0] = z0;
      r[i][1] = z1;
    }
  }

  __device__ __forceinline__ void store_rows(uint16_t* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int gi = tid + i * NT;
      if (G % NT == 0 || gi < G) {
        const int c8 = gi % (D / 8), rp = gi / (D / 8);
        *reinterpret_cast<uint4*>(dst + (2 * rp) * STRIDE + c8 * 8) = r[i][0];
        *reinterpret_cast<uint4*>(dst + (2 * rp + 1) * STRIDE + c8 * 8) = r[i][1];
      }
    }
  }

  __device__ __forceinline__ void store_trans(uint16_t* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int gi = tid + i * NT;
      if (G % NT == 0 || gi < G) {
        const int c8 = gi % (D / 8), rp = gi / (D / 8);
        const uint32_t x[4] = {r[i][0].x, r[i][0].y, r[i][0].z, r[i][0].w};
        const uint32_t y[4] = {r[i][1].x, r[i][1].y, r[i][1].z, r[i][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // (row 2rp, row 2rp+1) of dim c8*8+e: perm16 keeps the pair adjacent
          const uint32_t w = (e & 1) ? __builtin_amdgcn_perm(y[e / 2], x[e / 2], 0x07060302u)
                                     : __builtin_amdgcn_perm(y[e / 2], x[e / 2], 0x05040100u);
          *reinterpret_cast<uint32_t*>(dst + trans_index<ROWS>(c8 * 8 + e, 2 * rp)) = w;
        }
      }
    }
  }
};

}  // namespace dualkv
