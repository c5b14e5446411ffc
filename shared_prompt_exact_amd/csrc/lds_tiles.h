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
//    parity (D = 64: two 128-byte rows per 256 bytes), or 4 over the 4 rows
//    of each residue mod 4 (D = 32: four 64-byte rows per 256 bytes);
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
  if constexpr (D == 32) return (row >> 2) & 3;
  else if constexpr (D == 64) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
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

// The same transposed operand with k in natural order (slot j of half h <->
// row 8*h + j), for a product whose other operand is a plain row read: the
// two reads take rows 8h .. 8h+3 and 8h+4 .. 8h+7 of the step.  Each group of
// 16 lanes still reads four consecutive rows (four values of swz bits 2-3)
// by four consecutive chunks, so it stays free of bank conflicts.
template <int D>
__device__ __forceinline__ bf16x8 trans_operand_nat(const uint16_t* tile, int row0, int col0, int ks,
                                                    int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int hf = g >> 1, ib = (g & 1) * 16;
  const int col = col0 + ib + 4 * (s & 3);
  const int r0 = row0 + 16 * ks + 8 * hf + (s >> 2);
  const lds_short4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_as3*)(tile + tile_off<D>(r0, col)));
  const lds_short4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_as3*)(tile + tile_off<D>(r0 + 4, col)));
  const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
  const uint4 u = {x.x, x.y, y.x, y.y};
  return __builtin_bit_cast(bf16x8, u);
}

// ---- XOR-addressed operand reads -------------------------------------------
//
// In a swizzled tile the byte address of (row, chunk c) is
//   row * 2D + ((c ^ swz(row)) << 4),
// and since row * 2D has no bits inside the chunk field (bits 4 .. 4 +
// log2(D/8) - 1), that is  (row * 2D + (swz(row) << 4)) ^ (c << 4).  So a
// lane keeps ONE base address per row pattern and reaches every chunk with a
// single v_xor against a compile-time constant; tile, slot and 16-row steps
// (which leave swz unchanged) are immediate offsets of the LDS instruction.
// `base` values below are byte offsets from the start of LDS.

__device__ __forceinline__ const uint16_t* lds_at(const uint16_t* lds0, unsigned byte_off) {
  return reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(lds0) + byte_off);
}

// Base of the row operand for this lane: row `row`, wave half hf folded in
// (logical chunk 2*kk + hf is then base ^ (kk << 5)).
template <int D>
__device__ __forceinline__ unsigned row_base(int row, int hf) {
  return (unsigned)row * (2 * D) + (unsigned)((swz<D>(row) ^ hf) << 4);
}

// Row operand of k-step kk from a row base, at byte offset `imm` (tile/slot).
template <int D>
__device__ __forceinline__ bf16x8 row_operand_x(const uint16_t* lds0, unsigned base, int kk, unsigned imm) {
  return *reinterpret_cast<const bf16x8*>(lds_at(lds0, (base ^ ((unsigned)kk << 5)) + imm));
}

// Bases of the transposed operand (see trans_operand): the lane's first
// and second 8-row reads, column block 0, k-step 0.
template <int D>
__device__ __forceinline__ void trans_bases(int lane, unsigned& b0, unsigned& b1) {
  const int g = lane >> 4, s = lane & 15;
  const int hf = g >> 1, ib = (g & 1) * 16;
  const int col = ib + 4 * (s & 3);                  // 0 .. 31
  const int r0 = 4 * hf + (s >> 2);                  // 0 .. 7
  b0 = (unsigned)r0 * (2 * D) + (unsigned)((((col >> 3) ^ swz<D>(r0))) << 4) + (unsigned)((col & 7) * 2);
  const int r1 = r0 + 8;
  b1 = (unsigned)r1 * (2 * D) + (unsigned)((((col >> 3) ^ swz<D>(r1))) << 4) + (unsigned)((col & 7) * 2);
}

// Bases of the natural-order transposed operand (see trans_operand_nat).
template <int D>
__device__ __forceinline__ void trans_bases_nat(int lane, unsigned& b0, unsigned& b1) {
  const int g = lane >> 4, s = lane & 15;
  const int hf = g >> 1, ib = (g & 1) * 16;
  const int col = ib + 4 * (s & 3);                  // 0 .. 31
  const int r0 = 8 * hf + (s >> 2);                  // 0 .. 11
  b0 = (unsigned)r0 * (2 * D) + (unsigned)((((col >> 3) ^ swz<D>(r0))) << 4) + (unsigned)((col & 7) * 2);
  const int r1 = r0 + 4;
  b1 = (unsigned)r1 * (2 * D) + (unsigned)((((col >> 3) ^ swz<D>(r1))) << 4) + (unsigned)((col & 7) * 2);
}

// Transposed operand of column block cb (32 columns) and k-step ks from the
// bases above, at byte offset `imm`: 32-column blocks are chunk groups of 4,
// i.e. an XOR of (4*cb) << 4 = cb << 6; k-steps are 16 rows (an immediate).
template <int D>
__device__ __forceinline__ bf16x8 trans_operand_x(const uint16_t* lds0, unsigned b0, unsigned b1, int cb, int ks,
                                                  unsigned imm) {
  const unsigned x = (unsigned)cb << 6;
  const unsigned off = imm + (unsigned)ks * 16u * (2 * D);
  const lds_short4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_as3*)lds_at(lds0, (b0 ^ x) + off));
  const lds_short4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_as3*)lds_at(lds0, (b1 ^ x) + off));
  const u32x2 xa = __builtin_bit_cast(u32x2, a), yb = __builtin_bit_cast(u32x2, b);
  const uint4 u = {xa.x, xa.y, yb.x, yb.y};
  return __builtin_bit_cast(bf16x8, u);
}

// Per-lane global offset (bytes) of this lane's chunk in 1 KiB block `blk`
// of a tile whose rows are `row_bytes` apart: the lane lands at physical
// chunk lane % (D/8) of its row, so it fetches logical chunk
// (lane % (D/8)) ^ swz(row).  Valid for every tile of full rows.
template <int D>
__device__ __forceinline__ unsigned dma_lane_offset(int blk, int lane, unsigned row_bytes) {
  constexpr int CPR = D / 8, RPB = 64 / CPR;
  const int row = blk * RPB + lane / CPR;
  const int c = (lane % CPR) ^ swz<D>(row);
  return (unsigned)row * row_bytes + (unsigned)c * 16u;
}

// A wave-uniform pointer in scalar registers (the scalar base of a
// direct-to-LDS load) when the compiler cannot prove the uniformity.  Both
// halves go through unsigned 32-bit values: readfirstlane returns int, and a
// sign-extended low half would set the upper 32 bits.
__device__ __forceinline__ uint64_t join_halves(uint32_t lo, uint32_t hi) {
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (const uint16_t*)(uintptr_t)join_halves(lo, hi);
}

// One 1 KiB block of a tile by direct global->LDS load: global address
// `gbase` (wave-uniform, scalar) + this lane's offset, LDS destination
// `lds_byte` (wave-uniform).  No vector arithmetic on the address.
__device__ __forceinline__ void dma_block(const void* gbase, unsigned voff, unsigned lds_byte) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(gbase), "{m0}"(lds_byte));
}

}  // namespace dualkv
