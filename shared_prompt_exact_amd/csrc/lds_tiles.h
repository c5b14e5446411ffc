// LDS tiles fed by direct global->LDS loads, read as MFMA operands.
//
// A tile holds ROWS packed rows of one head (D bf16 each) row-major in
// LDS, 16-byte chunks XOR-swizzled per row: logical chunk c of row r sits
// at chunk c ^ swz<D>(r).  gfx950's LDS serves 256 bytes per clock over 64
// four-byte banks, so an access is conflict free when the 16-byte chunks
// that one clock serves land on 16 distinct positions modulo 256 bytes.
// One swizzle serves both operand reads:
//  * row operands (128-bit ds_read, 16 lanes per clock = 16 consecutive
//    rows at one logical chunk): swz takes 16 distinct values over 16
//    consecutive rows (D >= 128; rows are 256 B or more, so the position is
//    the chunk index mod 16), or 8 distinct values over the 8 rows of each
//    parity (D = 64: two 128-byte rows per 256 bytes);
//  * transposed operands (ds_read_b64_tr_b16, 32 lanes per clock = 4
//    consecutive rows x 4 consecutive chunks): the 4 rows differ in swz
//    bits 2-3 (D = 64: the two rows of each parity differ in bit 2), the 4
//    chunks in bits 0-1, so the 16 chunks read are distinct.
// Loading: global_load_lds_dwordx4 writes 64 lanes x 16 bytes = 1 KiB of
// LDS at a wave-uniform base, lane i at base + 16*i.  Lane i therefore
// fetches the global chunk that belongs at physical chunk i of its row.
// The loads complete asynchronously (counted by vmcnt); the kernels wait
// with explicit vmcnt counts and synchronize with a bare s_barrier so that
// tiles several stages ahead stay in flight.  The loads are issued as
// inline assembly: the compiler then does not know of the LDS DMA and does
// not drain it before every LDS read it cannot prove disjoint; the kernels'
// explicit waits are the only ordering they need.  Rows past the valid range
// re-read the last valid row: the values are finite and masked.
#pragma once

#include "mfma_common.h"

namespace dualkv {

typedef short lds_short4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) lds_short4 lds_short4_as3;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 64) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  else return ((row & 3) << 2) | ((row >> 2) & 3);
}

// Element offset of (row, col) in a swizzled tile with D columns.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ swz<D>(row))) << 3) + (col & 7);
}

// Wait until at most N vector-memory operations of this wave are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the memory fence of __syncthreads (which
// would drain every outstanding load).  LDS visibility is established by
// the explicit waits around it; the empty asm statements keep the compiler
// from moving memory operations across.
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads are done
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Issue this wave's share of a tile load: blocks [first, first + count) of
// the tile, each block RPB = 1024 / (2*D) rows.  `g` points at row 0 of the
// tile in global memory (head column already applied), `rs` is the row
// stride in elements, rows >= nvalid re-read row nvalid-1 (nvalid >= 1).
template <int D>
__device__ __forceinline__ void dma_rows(const uint16_t* __restrict__ g, int64_t rs, int nvalid,
                                         uint16_t* tile, int first_block, int count, int lane) {
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RPB = 64 / CPR;       // rows per 1 KiB block
#pragma unroll 4
  for (int b = 0; b < count; ++b) {
    const int blk = first_block + b;
    const int row = blk * RPB + lane / CPR;
    const int p = lane % CPR;
    const int c = p ^ swz<D>(row);
    const int src = row < nvalid ? row : nvalid - 1;
    const uint16_t* gp = g + (int64_t)src * rs + c * 8;
    // LDS base of the block in M0 (wave-uniform), 16 bytes per lane.
    const unsigned ldsaddr = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(tile + blk * 512));
    asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(gp), "{m0}"(ldsaddr));
  }
}

// Row operand: row `row`, k-step kk (16 columns), wave half hf.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* tile, int row, int kk, int hf) {
  return *reinterpret_cast<const bf16x8*>(tile + row * D + (((2 * kk + hf) ^ swz<D>(row)) << 3));
}

// Transposed operand for v_mfma_f32_32x32x16_bf16: A[i][k] = tile[row0 + k][col0 + i]
// for i < 32 (lane % 32) and the 16 k of step `ks`, with the k-slot order of
// a C tile reused as B operand (slot s of half h <-> row 8*(s/4) + 4*h + s%4).
template <int D>
__device__ __forceinline__ bf16x8 trans_operand(const uint16_t* tile, int row0, int col0, int ks,
                                                int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int hf = g >> 1, ib = (g & 1) * 16;
  const int col = col0 + ib + 4 * (s & 3);
  const int r0 = row0 + 16 * ks + 4 * hf + (s >> 2);
  const lds_short4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_as3*)(tile + tile_off<D>(r0, col)));
  const lds_short4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_as3*)(tile + tile_off<D>(r0 + 8, col)));
  const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
  const uint4 u = {x.x, x.y, y.x, y.y};
  return __builtin_bit_cast(bf16x8, u);
}

}  // namespace dualkv
