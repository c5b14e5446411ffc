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
// Tiling: a workgroup computes a BM x 128 block of C (BM = 256 with eight
// waves and a three-slot ring where the rows allow, else 128 with four
// waves and two slots), each wave 64 x 64 as 2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16; K advances 64 at a time through an LDS ring
// filled by direct global->LDS loads (the same swizzled tile layout as the
// attention kernels).  Both
// operands number their k-slots in the order of the attention kernels'
// transposed reads (half h of a 16-step holds k = 8*(j/4) + 4*h + j%4), so
// k-major tiles are read transposed and m- or n-major tiles with two
// 8-byte reads per operand.
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

// Tile of BM x 64*WN: waves of 64 x 32*WN (WN = 2: BM = 128 with four waves,
// a two-slot ring and two workgroups per CU, or BM = 256 with eight waves
// and a three-slot ring, tile loads two k-steps ahead; WN = 4: 256 x 256
// with eight waves of 64 x 128 and a two-slot ring, eight MFMAs per six
// operand reads).
template <int BM, int WN>
struct GemmCfg {
  static constexpr int GBN = 64 * WN;             // columns of C per workgroup
  static constexpr int NW = BM / 32;              // waves, each 64 x 32*WN
  static constexpr int NS = (BM == 256 && WN == 2) ? 3 : 2;    // ring slots
  static constexpr int A_ELEMS = BM * GBK, B_ELEMS = GBN * GBK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS = NS * STAGE * 2;      // bytes
  static constexpr int ABLK = A_ELEMS * 2 / 1024, BBLK = B_ELEMS * 2 / 1024;   // 1-KiB blocks
  static constexpr int APW = ABLK / NW, BPW = BBLK / NW;                        // per wave
  static_assert(ABLK % NW == 0 && BBLK % NW == 0, "tile blocks split evenly over the waves");
};

// A/B operand from an m- (or n-) major tile [rows][64 k]: row `row`,
// 16-step ks, wave half hf, k-slots in the transposed-read order.
__device__ __forceinline__ bf16x8 kslot_row_operand(const uint16_t* tile, int row, int ks, int hf) {
  const int c0 = 2 * ks, c1 = 2 * ks + 1;     // 16-byte chunks holding k = 16ks .. 16ks+15
  const uint16_t* p0 = tile + row * GBK + ((c0 ^ swz<GBK>(row)) << 3) + 4 * hf;
  const uint16_t* p1 = tile + row * GBK + ((c1 ^ swz<GBK>(row)) << 3) + 4 * hf;
  const uint2 a = *reinterpret_cast<const uint2*>(p0);
  const uint2 b = *reinterpret_cast<const uint2*>(p1);
  const uint4 u = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, u);
}

template <bool TA, bool TB, int BM, int WN>
__global__ void __launch_bounds__(BM * 2)
    gemm_bf16_kernel(int M, int N, int K, const uint16_t* __restrict__ A, int64_t lda,
                     const uint16_t* __restrict__ B, int64_t ldb, uint16_t* C, int64_t ldc,
                     const uint16_t* R, int64_t ldr, int tiles_n) {
  using G = GemmCfg<BM, WN>;
  constexpr int NS = G::NS, GBN = G::GBN;
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;     // 64 x 32*WN block of the wave
  const int bm = blockIdx.x / tiles_n, bn = blockIdx.x % tiles_n;
  const int m0 = bm * BM, n0 = bn * GBN;
  const int nk = (K + GBK - 1) / GBK;

  // this wave's share of the 1-KiB blocks of each tile
  auto issue = [&](int t) {
    uint16_t* As = lds + (t % NS) * G::STAGE;
    uint16_t* Bs = As + G::A_ELEMS;
    const int k0 = t * GBK;
    if constexpr (TA)   // [K][M]: 64 rows of k, BM m each
      dma_rows<BM>(A + (int64_t)k0 * lda + m0, lda, min(GBK, K - k0), As, wave * G::APW, G::APW, lane);
    else                // [M][K]: BM rows of m, 64 k each
      dma_rows<GBK>(A + (int64_t)m0 * lda + k0, lda, min(BM, M - m0), As, wave * G::APW, G::APW, lane);
    if constexpr (TB)   // [N][K]
      dma_rows<GBK>(B + (int64_t)n0 * ldb + k0, ldb, min(GBN, N - n0), Bs, wave * G::BPW, G::BPW, lane);
    else                // [K][N]
      dma_rows<GBN>(B + (int64_t)k0 * ldb + n0, ldb, min(GBK, K - k0), Bs, wave * G::BPW, G::BPW, lane);
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
  for (int t = 0; t < nk; ++t) {
    // tile t has landed once only the later tiles' loads (up to NS-2 of
    // them, APW + BPW instructions each) are pending
    if (NS == 3 && t + 1 < nk) wait_vmcnt<(NS - 2) * (G::APW + G::BPW)>();
    else wait_vmcnt<0>();
    block_sync();                              // everyone's; slot (t-1)%NS is free
    if (t + NS - 1 < nk) issue(t + NS - 1);
    uint16_t* As = lds + (t % NS) * G::STAGE;
    uint16_t* Bs = As + G::A_ELEMS;
    if constexpr (TA && !TB) {
      const int kv = K - t * GBK;              // valid k rows of this tile
      if (kv < GBK) {
        // rows kv..63 of both k-major tiles re-read row kv-1: zero them
        constexpr int CA = BM / 8, CB = GBN / 8;   // 16-byte chunks per row
        for (int i = tid; i < (GBK - kv) * (CA + CB); i += BM * 2) {
          const int r = kv + i / (CA + CB), c = i % (CA + CB);
          if (c < CA) *reinterpret_cast<uint4*>(As + r * BM + c * 8) = uint4{0, 0, 0, 0};
          else *reinterpret_cast<uint4*>(Bs + r * GBN + (c - CA) * 8) = uint4{0, 0, 0, 0};
        }
        block_sync();
      }
    }
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      bf16x8 a[2], b[WN];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int mr = wm * 64 + i * 32;
        if constexpr (TA) a[i] = trans_operand<BM>(As, 0, mr, ks, lane);
        else a[i] = kslot_row_operand(As, mr + l32, ks, hf);
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int nr = wn * 32 * WN + j * 32;
        if constexpr (TB) b[j] = kslot_row_operand(Bs, nr + l32, ks, hf);
        else b[j] = trans_operand<GBN>(Bs, 0, nr, ks, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
  }

  // C tile (i, j): lane column n, rows 8*(e/4) + 4*hf + e%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = n0 + wn * 32 * WN + j * 32 + l32;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
        if (m < M) {
          float x = acc[i][j][e];
          if (R) x += bf16_to_f32(R[(int64_t)m * ldr + n]);
          C[(int64_t)m * ldc + n] = f32_to_bf16(x);
        }
      }
    }
}

template <bool TA, bool TB, int BM, int WN>
hipError_t run_gemm(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                    int64_t ldc, const void* R, int64_t ldr, hipStream_t stream) {
  using G = GemmCfg<BM, WN>;
  static_assert(G::LDS <= 160 * 1024, "LDS budget");
  static const hipError_t attr = allow_lds(gemm_bf16_kernel<TA, TB, BM, WN>, G::LDS);
  if (attr != hipSuccess) return attr;
  const int tm = (M + BM - 1) / BM, tn = (N + G::GBN - 1) / G::GBN;
  return launch("gemm", gemm_bf16_kernel<TA, TB, BM, WN>, dim3((unsigned)(tm * tn)), dim3(BM * 2), G::LDS, stream, M,
                N, K, static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(B), ldb,
                static_cast<uint16_t*>(C), ldc, static_cast<const uint16_t*>(R), ldr, tn);
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
  // 16-byte global rows for the direct-to-LDS loads
  if (lda % 8 != 0 || ldb % 8 != 0) return 0;
  if ((int64_t)((M + 127) / 128) * ((N + GBN - 1) / GBN) >= ((int64_t)1 << 31)) return 0;
  return 1;
}

hipError_t launch_gemm(bool ta, bool tb, int M, int N, int K, const void* A, int64_t lda, const void* B,
                       int64_t ldb, void* C, int64_t ldc, const void* R, int64_t ldr, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (ta && tb) return hipErrorInvalidValue;
  const bool tall = use_tall(ta, M, N), wide = use_wide(ta, M, N);
  if (ta)
    return wide ? run_gemm<true, false, 256, 4>(M, N, K, A, lda, B, ldb, C, ldc, R, ldr, stream)
         : tall ? run_gemm<true, false, 256, 2>(M, N, K, A, lda, B, ldb, C, ldc, R, ldr, stream)
                : run_gemm<true, false, 128, 2>(M, N, K, A, lda, B, ldb, C, ldc, R, ldr, stream);
  if (tb)
    return wide ? run_gemm<false, true, 256, 4>(M, N, K, A, lda, B, ldb, C, ldc, R, ldr, stream)
         : tall ? run_gemm<false, true, 256, 2>(M, N, K, A, lda, B, ldb, C, ldc, R, ldr, stream)
                : run_gemm<false, true, 128, 2>(M, N, K, A, lda, B, ldb, C, ldc, R, ldr, stream);
  return wide ? run_gemm<false, false, 256, 4>(M, N, K, A, lda, B, ldb, C, ldc, R, ldr, stream)
       : tall ? run_gemm<false, false, 256, 2>(M, N, K, A, lda, B, ldb, C, ldc, R, ldr, stream)
              : run_gemm<false, false, 128, 2>(M, N, K, A, lda, B, ldb, C, ldc, R, ldr, stream);
}

}  // namespace dualkv
