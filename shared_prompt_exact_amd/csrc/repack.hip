// Row repack between the replicated N(P+R) layout and the packed P+NR
// layout ("DualKV: Shared-Prompt Flash Attention ...", arXiv 2605.15422,
// Abstract: the data pipeline keeps one copy of the shared prompt).
//
// Pure data movement, bound by HBM bandwidth: every destination row is
// copied from one source row.  A workgroup copies whole rows with the
// widest access the row size and the pointer alignment allow (16, 8, 4 or
// 1 bytes per lane), so a row of a few KiB becomes fully coalesced
// 128-bit loads and stores.
#include "common.h"

namespace dualkv {
namespace {

__device__ __forceinline__ int64_t src_row(int64_t row, int N, int P, int R, int direction) {
  if (direction == DUALKV_GATHER) {
    // packed row -> replicated row; the prompt comes from copy 0
    if (row < P) return row;
    int64_t rel = row - P;
    int64_t n = rel / R, r = rel - n * R;
    return n * (int64_t)(P + R) + P + r;
  }
  // replicated row -> packed row; the prompt is broadcast to every copy
  int64_t n = row / (P + R), i = row - n * (int64_t)(P + R);
  return i < P ? i : (int64_t)P + n * R + (i - P);
}

template <typename V>
__global__ void __launch_bounds__(256) repack_kernel(const V* __restrict__ src, V* __restrict__ dst,
                                                     int64_t row_elems, int64_t n_rows, int N, int P,
                                                     int R, int direction) {
  // rows_per_block rows share one workgroup when rows are short
  const int64_t rows_per_iter = row_elems >= 256 ? 1 : (256 / row_elems);
  const int64_t lane_row = row_elems >= 256 ? 0 : threadIdx.x / row_elems;
  const int64_t lane_elem = row_elems >= 256 ? threadIdx.x : threadIdx.x % row_elems;
  const int64_t step_elem = row_elems >= 256 ? 256 : row_elems;
  if (lane_row >= rows_per_iter) return;
  for (int64_t row0 = (int64_t)blockIdx.x * rows_per_iter; row0 < n_rows;
       row0 += (int64_t)gridDim.x * rows_per_iter) {
    int64_t row = row0 + lane_row;
    if (row >= n_rows) break;
    int64_t s = src_row(row, N, P, R, direction);
    const V* sp = src + s * row_elems;
    V* dp = dst + row * row_elems;
    for (int64_t e = lane_elem; e < row_elems; e += step_elem) dp[e] = sp[e];
  }
}

template <typename V>
hipError_t go(const void* src, void* dst, int64_t row_bytes, int64_t n_rows, int N, int P, int R,
              int direction, hipStream_t stream) {
  int64_t row_elems = row_bytes / (int64_t)sizeof(V);
  int64_t rows_per_iter = row_elems >= 256 ? 1 : 256 / row_elems;
  int64_t blocks = (n_rows + rows_per_iter - 1) / rows_per_iter;
  if (blocks > 256 * 64) blocks = 256 * 64;
  return launch("repack", repack_kernel<V>, dim3((unsigned)blocks), dim3(256), 0, stream,
                static_cast<const V*>(src), static_cast<V*>(dst), row_elems, n_rows, N, P, R,
                direction);
}

}  // namespace

hipError_t launch_repack(const void* src, void* dst, int64_t row_bytes, int N, int P, int R,
                         int direction, hipStream_t stream) {
  int64_t n_rows = direction == DUALKV_GATHER ? (int64_t)P + (int64_t)N * R : (int64_t)N * (P + R);
  if (n_rows == 0) return hipSuccess;
  uintptr_t a = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
  if (row_bytes % 16 == 0 && a % 16 == 0)
    return go<uint4>(src, dst, row_bytes, n_rows, N, P, R, direction, stream);
  if (row_bytes % 8 == 0 && a % 8 == 0)
    return go<uint2>(src, dst, row_bytes, n_rows, N, P, R, direction, stream);
  if (row_bytes % 4 == 0 && a % 4 == 0)
    return go<uint32_t>(src, dst, row_bytes, n_rows, N, P, R, direction, stream);
  return go<uint8_t>(src, dst, row_bytes, n_rows, N, P, R, direction, stream);
}

}  // namespace dualkv
