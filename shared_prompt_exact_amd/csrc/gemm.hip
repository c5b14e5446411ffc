// bf16 GEMM on gfx950 matrix cores, for the projections of a packed
// transformer layer (the token-wise work that runs on P+NR packed rows
// instead of N(P+R) replicated rows).
//
//   C[m][n] = sum_k A[m][k] * B[k][n]  (+ R[m][n]),  fp32 accumulation,
//   bf16 inputs and output, all row-major with leading dimensions.
// A is stored [M][K] (lda >= K) or, with TA, transposed as [K][M];
// B is stored [K][N] or, with TB, transposed as [N][K].  The three forms a
// linear layer needs: y = x W (NN), dx = dy W^T (NT), dW = x^T dy (TN).
//
// Tiling: a workgroup computes a BM x 64*WN block of C with BM/32 waves of
// 64 x 32*WN, as 2 x WN tiles of v_mfma_f32_32x32x16_bf16: 256 x 256 (eight
// waves, a two-slot ring of 64-deep k tiles) where the shape allows, else
// 256 x 128 (three slots) or 128 x 128 (four waves, two slots).  K advances
// through an LDS ring filled by direct global->LDS loads, in the swizzled
// tile layout of the attention kernels.  Operands: an m- or n-major tile
// ([M][K] A, [N][K] B) is read by rows, one 16-byte read per operand, k in
// natural order; a k-major tile is read with the transposing LDS read.  In
// x W (only B k-major) that read takes k in natural order too; in x^T dy
// (both k-major) both take the k-slot order of the attention kernels' C-tile
// reuse (half h of a 16-step holds k = 8*(j/4) + 4*h + j%4).  The wave forms
// C^T tiles (B^T A^T), so each lane holds runs of four columns of one row of
// C and the epilogue stores (and reads the residual) 8 bytes at a time.
//
// Bounds: rows of an [M][K] A tile or [N][K] B tile beyond M (N) re-read
// the last valid row and their results are not stored.  Tiles whose rows
// are k (TA, or B without TB) need whole 128-column blocks of M (N); tiles
// whose columns are k need K % 64 == 0; with TA and no TB (both tiles
// k-major, the weight-gradient form) a partial last k tile is zeroed in
// LDS, so K is free.  The host launcher checks these.
#include "lds_tiles.h"

namespace dualkv {

namespace {

constexpr int GBK = 64;

template <int V>
struct IntC {
  static constexpr int value = V;
};

constexpr int kWideBK = 64, kWideNS = 2;

// Tile of BM x 64*WN: waves of 64 x 32*WN (WN = 2: BM = 128 with four waves,
// a two-slot ring and two workgroups per CU, or BM = 256 with eight waves
// and a three-slot ring, tile loads two k-steps ahead; WN = 4: 256 x 256
// with eight waves of 64 x 128 and a two-slot ring, eight MFMAs per six
// operand reads).
template <int BM, int WN>
struct GemmCfg {
  static constexpr int GBN = 64 * WN;             // columns of C per workgroup
  static constexpr int NW = BM / 32;              // waves, each 64 x 32*WN
  static constexpr int BK = WN == 4 ? kWideBK : GBK;   // k per ring slot
  static constexpr int NS = WN == 4 ? kWideNS : (BM == 256 ? 3 : 2);    // ring slots
  static constexpr int A_ELEMS = BM * BK, B_ELEMS = GBN * BK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS = NS * STAGE * 2;      // bytes
  static constexpr int ABLK = A_ELEMS * 2 / 1024, BBLK = B_ELEMS * 2 / 1024;   // 1-KiB blocks
  static constexpr int APW = ABLK / NW, BPW = BBLK / NW;                        // per wave
  static_assert(ABLK % NW == 0 && BBLK % NW == 0, "tile blocks split evenly over the waves");
};

template <bool TA, bool TB, int BM, int WN>
__global__ void __launch_bounds__(BM * 2)
    gemm_bf16_kernel(int M, int N, int K, GemmParts P, int tiles_n, int vec) {
  using G = GemmCfg<BM, WN>;
  constexpr int NS = G::NS, GBN = G::GBN, BK = G::BK;
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;     // 64 x 32*WN block of the wave
  int bm, bn;
  gemm_tile_of(blockIdx.x, gridDim.x / tiles_n, tiles_n, bm, bn);
  const int m0 = bm * BM;
  // column part of this tile (all of C when the parts split k)
  int cp = 0;
  if (!P.ksplit)
    while (cp + 1 < P.n && bn * GBN >= P.lo[cp + 1]) ++cp;
  const int c_lo = P.ksplit ? 0 : P.lo[cp];
  const int n0 = bn * GBN - c_lo;              // first column inside the part
  const int Nl = P.ksplit ? N : P.lo[cp + 1] - c_lo;
  const int nk = (K + BK - 1) / BK;

  // operands of k tile t: its part, and the tile's first k inside the part
  struct Ops { const uint16_t* A; int64_t lda; const uint16_t* B; int64_t ldb; int k0, Kl, kp; };
  auto ops = [&](int t) {
    int kp = 0;
    if (P.ksplit)
      while (kp + 1 < P.n && t * BK >= P.lo[kp + 1]) ++kp;
    const int k_lo = P.ksplit ? P.lo[kp] : 0;
    const int bp = P.ksplit ? kp : cp;
    return Ops{P.A[kp], P.lda[kp], P.B[bp], P.ldb[bp], t * BK - k_lo, P.ksplit ? P.lo[kp + 1] - k_lo : K, kp};
  };

  // Operand addresses: one XOR-derived base per lane and operand pattern
  // (lds_tiles.h), ring slots and the second 32-row (column) block as
  // immediates; the wave's row (column) block is folded into the base.
  constexpr unsigned A_BYTES = G::A_ELEMS * 2, STAGE_BYTES = G::STAGE * 2;
  unsigned abase, a0, a1, bbase, b0, b1;
  if constexpr (TA) {
    trans_bases<BM>(lane, a0, a1);
    a0 ^= (unsigned)(2 * wm) << 6;
    a1 ^= (unsigned)(2 * wm) << 6;
  } else {
    abase = row_base<BK>(wm * 64 + l32, hf);
  }
  if constexpr (TB) {
    bbase = A_BYTES + row_base<BK>(wn * 32 * WN + l32, hf);
  } else {
    if constexpr (TA) trans_bases<GBN>(lane, b0, b1);
    else trans_bases_nat<GBN>(lane, b0, b1);
    b0 = A_BYTES + (b0 ^ ((unsigned)(wn * WN) << 6));
    b1 = A_BYTES + (b1 ^ ((unsigned)(wn * WN) << 6));
  }

  // Tile loads: a full tile takes a scalar base and per-lane offsets fixed
  // for the kernel; a partial one (rows past M or N, k past K) re-reads its
  // last valid row through dma_rows.
  const bool a_rows_full = TA || m0 + BM <= M;
  const bool b_rows_full = !TB || n0 + GBN <= Nl;
  // per-lane offsets of the wave's blocks for the leading dimensions of the
  // current part (k parts may differ; they are recomputed when it changes)
  unsigned avoff[G::APW], bvoff[G::BPW];
  auto lane_offsets = [&](int64_t lda, int64_t ldb) {
#pragma unroll
    for (int j = 0; j < G::APW; ++j)
      avoff[j] = TA ? dma_lane_offset<BM>(wave * G::APW + j, lane, (unsigned)(lda * 2))
                    : dma_lane_offset<BK>(wave * G::APW + j, lane, (unsigned)(lda * 2));
#pragma unroll
    for (int j = 0; j < G::BPW; ++j)
      bvoff[j] = TB ? dma_lane_offset<BK>(wave * G::BPW + j, lane, (unsigned)(ldb * 2))
                    : dma_lane_offset<GBN>(wave * G::BPW + j, lane, (unsigned)(ldb * 2));
  };
  int cur_kp = 0;
  lane_offsets(P.lda[0], P.ldb[P.ksplit ? 0 : cp]);
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  auto issue = [&](int t) {
    uint16_t* As = lds + (t % NS) * G::STAGE;
    uint16_t* Bs = As + G::A_ELEMS;
    const unsigned adst = lds0 + (unsigned)((t % NS) * STAGE_BYTES) + (unsigned)(wave * G::APW) * 1024u;
    const unsigned bdst = adst - (unsigned)(wave * G::APW) * 1024u + A_BYTES + (unsigned)(wave * G::BPW) * 1024u;
    const Ops o = ops(t);
    if (o.kp != cur_kp) {                     // tiles are issued in k order: parts only advance
      lane_offsets(o.lda, o.ldb);
      cur_kp = o.kp;
    }
    const int k0 = o.k0;
    const bool k_full = k0 + BK <= o.Kl;
    if constexpr (TA) {   // [K][M]: 64 rows of k, BM m each
      const uint16_t* g = uniform_ptr(o.A + (int64_t)k0 * o.lda + m0);
      if (k_full) {
#pragma unroll
        for (int j = 0; j < G::APW; ++j) dma_block(g, avoff[j], adst + j * 1024u);
      } else {
        dma_rows<BM>(g, o.lda, min(BK, o.Kl - k0), As, wave * G::APW, G::APW, lane);
      }
    } else {              // [M][K]: BM rows of m, 64 k each
      const uint16_t* g = uniform_ptr(o.A + (int64_t)m0 * o.lda + k0);
      if (a_rows_full) {
#pragma unroll
        for (int j = 0; j < G::APW; ++j) dma_block(g, avoff[j], adst + j * 1024u);
      } else {
        dma_rows<BK>(g, o.lda, min(BM, M - m0), As, wave * G::APW, G::APW, lane);
      }
    }
    if constexpr (TB) {   // [N][K]
      const uint16_t* g = uniform_ptr(o.B + (int64_t)n0 * o.ldb + k0);
      if (b_rows_full) {
#pragma unroll
        for (int j = 0; j < G::BPW; ++j) dma_block(g, bvoff[j], bdst + j * 1024u);
      } else {
        dma_rows<BK>(g, o.ldb, min(GBN, Nl - n0), Bs, wave * G::BPW, G::BPW, lane);
      }
    } else {              // [K][N]
      const uint16_t* g = uniform_ptr(o.B + (int64_t)k0 * o.ldb + n0);
      if (k_full) {
#pragma unroll
        for (int j = 0; j < G::BPW; ++j) dma_block(g, bvoff[j], bdst + j * 1024u);
      } else {
        dma_rows<GBN>(g, o.ldb, min(BK, o.Kl - k0), Bs, wave * G::BPW, G::BPW, lane);
      }
    }
  };

  f32x16 acc[2][WN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < nk) issue(t);
  // one k tile; unrolled by the ring depth, so the slot is a compile-time
  // constant and every operand read is a base XOR plus an immediate
  auto step = [&](int t, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    constexpr unsigned SO = SLOT * STAGE_BYTES;
    // tile t has landed once only the later tiles' loads (up to NS-2 of
    // them, APW + BPW instructions each) are pending
    if (NS >= 3 && t + NS - 2 < nk) wait_vmcnt<(NS >= 3 ? NS - 2 : 0) * (G::APW + G::BPW)>();
    else wait_vmcnt<0>();
    block_sync();                              // everyone's; slot (t-1)%NS is free
    if (t + NS - 1 < nk) issue(t + NS - 1);
    if constexpr (TA && !TB) {
      uint16_t* As = lds + SLOT * G::STAGE;
      uint16_t* Bs = As + G::A_ELEMS;
      const Ops o = ops(t);
      const int kv = o.Kl - o.k0;             // valid k rows of this tile
      if (kv < BK) {
        // rows kv..63 of both k-major tiles re-read row kv-1: zero them
        constexpr int CA = BM / 8, CB = GBN / 8;   // 16-byte chunks per row
        for (int i = tid; i < (BK - kv) * (CA + CB); i += BM * 2) {
          const int r = kv + i / (CA + CB), c = i % (CA + CB);
          if (c < CA) *reinterpret_cast<uint4*>(As + r * BM + c * 8) = uint4{0, 0, 0, 0};
          else *reinterpret_cast<uint4*>(Bs + r * GBN + (c - CA) * 8) = uint4{0, 0, 0, 0};
        }
        block_sync();
      }
    }
    unsigned ab = abase, x0 = a0, x1 = a1, bb = bbase, y0 = b0, y1 = b1;
    if constexpr (TA) asm volatile("" : "+v"(x0), "+v"(x1));
    else asm volatile("" : "+v"(ab));
    if constexpr (TB) asm volatile("" : "+v"(bb));
    else asm volatile("" : "+v"(y0), "+v"(y1));
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 a[2], b[WN];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (TA) a[i] = trans_operand_x<BM>(lds, x0, x1, i, ks, SO);
        else a[i] = row_operand_x<BK>(lds, ab, ks, SO + (unsigned)(i * 32 * BK * 2));
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        if constexpr (TB) b[j] = row_operand_x<BK>(lds, bb, ks, SO + (unsigned)(j * 32 * BK * 2));
        else b[j] = trans_operand_x<GBN>(lds, y0, y1, j, ks, SO);   // natural k order unless TA
      }
      // the product is formed transposed (C^T tile = B^T A^T), so that a
      // lane holds four consecutive columns of C in each register group
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = mfma32(b[j], a[i], acc[i][j]);
    }
  };
  static_assert(NS == 2 || NS == 3, "ring of two or three, unrolled by its depth");
  int t = 0;
  for (; t + NS <= nk; t += NS) {
    step(t, IntC<0>{});
    step(t + 1, IntC<1>{});
    if constexpr (NS == 3) step(t + 2, IntC<2 % NS>{});
  }
  if (t < nk) step(t, IntC<0>{});
  if constexpr (NS == 3)
    if (t + 1 < nk) step(t + 1, IntC<1>{});

  // C^T tile (i, j): lane row m, columns 8*(e/4) + 4*hf + e%4; four
  // consecutive columns go out (and the residual comes in) as 8 bytes
  uint16_t* C = P.C[cp];
  const uint16_t* R = P.R[cp];
  const int64_t ldc = P.ldc[cp], ldr = P.ldr[cp];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * 64 + i * 32 + l32;
    if (m >= M) continue;
    uint16_t* crow = C + (int64_t)m * ldc;
    const uint16_t* rrow = R ? R + (int64_t)m * ldr : nullptr;
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 32 * WN + j * 32 + 8 * q + 4 * hf;   // column inside the part
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[i][j][4 * q + e];
        if (vec && n + 3 < Nl) {
          if (rrow) {
            const uint2 r = *reinterpret_cast<const uint2*>(rrow + n);
            x[0] += __uint_as_float(r.x << 16);
            x[1] += __uint_as_float(r.x & 0xffff0000u);
            x[2] += __uint_as_float(r.y << 16);
            x[3] += __uint_as_float(r.y & 0xffff0000u);
          }
          uint2 o;
          o.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
          o.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
          *reinterpret_cast<uint2*>(crow + n) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < Nl) crow[n + e] = f32_to_bf16(x[e] + (rrow ? bf16_to_f32(rrow[n + e]) : 0.f));
        }
      }
  }
}

template <bool TA, bool TB, int BM, int WN>
hipError_t run_gemm(int M, int N, int K, const GemmParts& P, hipStream_t stream) {
  using G = GemmCfg<BM, WN>;
  static_assert(G::LDS <= 160 * 1024, "LDS budget");
  static const hipError_t attr = allow_lds(gemm_bf16_kernel<TA, TB, BM, WN>, G::LDS);
  if (attr != hipSuccess) return attr;
  const int tm = (M + BM - 1) / BM, tn = (N + G::GBN - 1) / G::GBN;
  // 8-byte epilogue accesses need 8-byte aligned rows of every C (and R)
  int vec = 1;
  for (int j = 0; j < (P.ksplit ? 1 : P.n); ++j)
    vec &= P.ldc[j] % 4 == 0 && reinterpret_cast<uintptr_t>(P.C[j]) % 8 == 0 &&
           (!P.R[j] || (P.ldr[j] % 4 == 0 && reinterpret_cast<uintptr_t>(P.R[j]) % 8 == 0));
  return launch("gemm", gemm_bf16_kernel<TA, TB, BM, WN>, dim3((unsigned)(tm * tn)), dim3(BM * 2), G::LDS, stream, M,
                N, K, P, tn, vec);
}

constexpr int GBN = 128;   // the narrowest tile's columns: the shape rules below

// The 256-row tile where the rows allow it: whole 256-row blocks when A is
// k-major; otherwise enough rows that 256-row blocks fill the chip.
bool use_tall(bool ta, int M, int N) {
  if (ta) return M % 256 == 0;
  return (int64_t)((M + 255) / 256) * ((N + GBN - 1) / GBN) >= 512;
}

// The 256 x 256 tile: a tall tile whose columns come in whole 256-wide
// blocks, with at least one block per CU.
bool use_wide(bool ta, int M, int N) {
  return use_tall(ta, M, N) && N % 256 == 0 && (int64_t)((M + 255) / 256) * (N / 256) >= 256;
}

}  // namespace

int gemm_shape_ok(bool ta, bool tb, int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0) return 0;
  if (ta ? lda < M : lda < K) return 0;
  if (tb ? ldb < K : ldb < N) return 0;
  if (ldc < N) return 0;
  if (ta && tb) return 0;
  if (K == 0) return 1;                        // C = R (or 0): no operand is read
  if (ta && M % 128 != 0) return 0;            // k-major A: whole 128-wide m blocks
  if (!tb && N % GBN != 0) return 0;           // k-major B: whole 128-wide n blocks
  if (!(ta && !tb) && K % GBK != 0) return 0;  // k along tile columns: whole 64-wide k blocks
  // 16-byte global rows for the direct-to-LDS loads, whose per-lane byte
  // offsets inside a tile (up to 256 rows) are 32-bit
  if (lda % 8 != 0 || ldb % 8 != 0) return 0;
  if (lda >= ((int64_t)1 << 22) || ldb >= ((int64_t)1 << 22)) return 0;
  if ((int64_t)((M + 127) / 128) * ((N + GBN - 1) / GBN) >= ((int64_t)1 << 31)) return 0;
  return 1;
}

hipError_t launch_gemm_parts(bool ta, bool tb, int M, int N, int K, const GemmParts& P, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (ta && tb) return hipErrorInvalidValue;
  const bool tall = use_tall(ta, M, N), wide = use_wide(ta, M, N);
  if (ta)
    return wide ? run_gemm<true, false, 256, 4>(M, N, K, P, stream)
         : tall ? run_gemm<true, false, 256, 2>(M, N, K, P, stream)
                : run_gemm<true, false, 128, 2>(M, N, K, P, stream);
  if (tb)
    return wide ? run_gemm<false, true, 256, 4>(M, N, K, P, stream)
         : tall ? run_gemm<false, true, 256, 2>(M, N, K, P, stream)
                : run_gemm<false, true, 128, 2>(M, N, K, P, stream);
  return wide ? run_gemm<false, false, 256, 4>(M, N, K, P, stream)
       : tall ? run_gemm<false, false, 256, 2>(M, N, K, P, stream)
              : run_gemm<false, false, 128, 2>(M, N, K, P, stream);
}

hipError_t launch_gemm(bool ta, bool tb, int M, int N, int K, const void* A, int64_t lda, const void* B,
                       int64_t ldb, void* C, int64_t ldc, const void* R, int64_t ldr, hipStream_t stream) {
  GemmParts P{};
  P.n = 1;
  P.ksplit = 0;
  P.lo[0] = 0;
  P.lo[1] = N;
  P.A[0] = static_cast<const uint16_t*>(A);
  P.lda[0] = lda;
  P.B[0] = static_cast<const uint16_t*>(B);
  P.ldb[0] = ldb;
  P.C[0] = static_cast<uint16_t*>(C);
  P.ldc[0] = ldc;
  P.R[0] = static_cast<const uint16_t*>(R);
  P.ldr[0] = ldr;
  return launch_gemm_parts(ta, tb, M, N, K, P, stream);
}

}  // namespace dualkv
