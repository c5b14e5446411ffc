// Shared device/host definitions for the shared-prompt attention kernels
// (gfx950 only).  The packed layout, positions, masks and GQA mapping are
// those documented in include/dualkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "dualkv.h"

namespace dualkv {

// Validated problem description passed by value to every kernel.  In a
// launch over several prompt groups, N, P, R, T and valid_len describe one
// group (the kernels derive them per workgroup, see group_problem) and Tld
// counts the rows of all groups: LSE, Delta and their kin are [H, Tld].
struct Problem {
  int N, P, R;          // responses, prompt length, padded response length
  int Hq, Hkv, D;       // heads and head dim
  int g;                // Hq / Hkv
  int W;                // window (<= 0: none)
  int T;                // P + N*R packed rows
  int Tld;              // rows of the whole launch (leading dim of [H, rows] arrays)
  float scale;          // softmax scale (> 0)
  const int32_t* valid_len;  // device [N] or nullptr
};

// Prompt groups of one launch.  Group i holds packed rows row0[i] ..
// row0[i] + P[i] + N[i]*R[i] - 1 (its own prompt, then its N[i] responses),
// and its valid lengths start at entry vl0[i] of the launch's array.
constexpr int kMaxGroups = 32;
struct Groups {
  int n;
  int N[kMaxGroups], P[kMaxGroups], R[kMaxGroups];
  int row0[kMaxGroups], vl0[kMaxGroups];
};

// The problem of group gi (rows relative to the group's row 0).
__host__ __device__ inline Problem group_problem(const Problem& base, const Groups& G, int gi) {
  Problem p = base;
  p.N = G.N[gi];
  p.P = G.P[gi];
  p.R = G.R[gi];
  p.T = p.P + p.N * p.R;
  p.valid_len = base.valid_len ? base.valid_len + G.vl0[gi] : nullptr;
  return p;
}

// Order of a launch's work items across its groups.  Each group lists its
// items longest first; the launch cuts every group's list into at most
// kMaxChunks / n chunks of consecutive items and runs the chunks of all
// groups by decreasing cost of their first (longest) item, so the short
// items of every group meet at the end of the launch instead of each
// group's tail sitting between the next group's long items.  Chunk i covers
// launch positions [start[i], start[i+1]) and holds items loc[i] .. of
// group grp[i].
constexpr int kMaxChunks = 48;
struct LaunchOrder {
  int n;
  int start[kMaxChunks + 1];
  int loc[kMaxChunks];
  uint8_t grp[kMaxChunks];
};

// Group and item of launch position x (a binary search over at most
// kMaxChunks entries, scalar registers only).
__device__ __forceinline__ int order_lookup(const LaunchOrder& o, int x, int& item) {
  int lo = 0, hi = o.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (o.start[mid] <= x) lo = mid; else hi = mid - 1;
  }
  item = o.loc[lo] + (x - o.start[lo]);
  return o.grp[lo];
}

// Builds the order from the groups' item counts and a cost of item j of
// group i (cost(i, j) non-increasing in j).  One group keeps its own order.
// Equal costs keep group order (stable sort).
template <class Cost>
LaunchOrder make_order(const int64_t* count, int ngroups, Cost cost) {
  LaunchOrder o{};
  struct Chunk { double cost; int g, loc, len; };
  Chunk ch[kMaxChunks];
  int nc = 0;
  // one group: a single chunk, the group's own order
  const int per = ngroups > 1 ? kMaxChunks / ngroups : 1;
  for (int i = 0; i < ngroups; ++i) {
    const int64_t m = count[i];
    const int64_t k = m < per ? m : per;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t a = m * j / k, b = m * (j + 1) / k;
      if (b > a) ch[nc++] = Chunk{cost(i, (int)a), i, (int)a, (int)(b - a)};
    }
  }
  if (nc == 0) ch[nc++] = Chunk{0.0, 0, 0, 0};
  for (int i = 1; i < nc; ++i)   // stable insertion sort, decreasing cost
    for (int j = i; j > 0 && ch[j - 1].cost < ch[j].cost; --j) {
      const Chunk t = ch[j];
      ch[j] = ch[j - 1];
      ch[j - 1] = t;
    }
  o.n = nc;
  int pos = 0;
  for (int i = 0; i < nc; ++i) {
    o.start[i] = pos;
    o.loc[i] = ch[i].loc;
    o.grp[i] = (uint8_t)ch[i].g;
    pos += ch[i].len;
  }
  o.start[nc] = pos;
  return o;
}

// Logical blocks of a launch per group: group i owns off[i+1] - off[i]
// blocks; `ord` places them in the launch.
struct GroupBlocks {
  int off[kMaxGroups + 1];
  int nbP[kMaxGroups], nbR[kMaxGroups];   // prompt / response row blocks (query-parallel kernels)
  LaunchOrder ord;
};

// Cost (visible keys of its last query) of row block j of a group in the
// query-parallel kernels' order (decode_block): response blocks from the
// last down, then prompt blocks from the last down.
inline double row_block_cost(int N, int P, int R, int W, int BM, int nbP, int nbR, int j) {
  int64_t q_end;
  if (j < (int64_t)N * nbR) {
    const int rb = nbR - 1 - j / N;
    q_end = (int64_t)P + std::min<int64_t>((int64_t)(rb + 1) * BM, R);
  } else {
    const int pb = nbP - 1 - (j - N * nbR);
    q_end = std::min<int64_t>((int64_t)(pb + 1) * BM, P);
  }
  return (double)(W > 0 ? std::min<int64_t>(q_end, (int64_t)W + BM - 1) : q_end);
}

__device__ __forceinline__ int resp_valid(const Problem& pr, int n) {
  if (pr.valid_len == nullptr) return pr.R;
  int L = pr.valid_len[n];
  return L < 0 ? 0 : (L > pr.R ? pr.R : L);
}

// bf16 <-> fp32 on raw 16-bit patterns (round to nearest even; inputs of
// these kernels are finite, NaN is kept quiet).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Opt-in launch profiler (profile.hip): brackets launches with HIP events.
bool profiling_on();
int profile_begin(const char* name, hipStream_t stream);
void profile_end(int slot, hipStream_t stream);

// Launch a kernel and return the runtime's status for that launch (the
// status of hipLaunchKernel itself, not a stale error of an earlier call).
// `name` labels the launch for the profiler.
template <typename... KArgs, typename... Args>
static inline hipError_t launch(const char* name, void (*kern)(KArgs...), dim3 grid, dim3 block,
                                size_t shmem, hipStream_t stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  auto go = [&](KArgs... conv) -> hipError_t {
    void* ptrs[] = {static_cast<void*>(&conv)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, shmem, stream);
  };
  const int slot = profiling_on() ? profile_begin(name, stream) : -1;
  const hipError_t e = go(static_cast<KArgs>(args)...);
  if (slot >= 0) profile_end(slot, stream);
  return e;
}

// Validates a group table (1..kMaxGroups well-formed entries, at most
// 2^30 packed rows); returns a DUALKV_* status and the packed row count.
int check_groups(const dualkv_group* groups, int32_t n, int64_t* rows);

// Up to three GEMMs of one launch (gemm.hip).  Either the parts are column
// ranges [lo[j], lo[j+1]) of the output that share A, each with its own B,
// C and residual R (x Wk and x Wv side by side), or (ksplit) they are k
// ranges that share C and R, C = R + sum_j A_j B_j accumulated in fp32 (the
// input gradient of several projections of one input).  Part widths are
// whole column tiles (256) or whole k tiles (64); the launcher of one GEMM
// is the one-part case.
constexpr int kMaxGemmParts = 3;
struct GemmParts {
  int n, ksplit;
  int lo[kMaxGemmParts + 1];
  const uint16_t* A[kMaxGemmParts];
  const uint16_t* B[kMaxGemmParts];
  uint16_t* C[kMaxGemmParts];
  const uint16_t* R[kMaxGemmParts];
  int64_t lda[kMaxGemmParts], ldb[kMaxGemmParts], ldc[kMaxGemmParts], ldr[kMaxGemmParts];
};

// ---- launchers implemented in the kernel translation units -------------
hipError_t launch_repack(const void* src, void* dst, int64_t row_bytes, int N, int P, int R,
                         int direction, hipStream_t stream);

// `pr` carries the launch-wide fields (heads, dims, window, scale, Tld,
// valid lengths); `G` the groups.
hipError_t launch_fwd_scalar(const Problem& pr, const Groups& G, int dtype, const void* q,
                             const void* k, const void* v, void* o, float* lse, hipStream_t stream);
hipError_t launch_bwd_scalar(const Problem& pr, const Groups& G, int dtype, const void* q,
                             const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, float* delta,
                             hipStream_t stream);

bool fwd_mfma_supported(const Problem& pr, const Groups& G);
hipError_t launch_fwd_mfma(const Problem& pr, const Groups& G, const void* q, const void* k,
                           const void* v, void* o, float* lse, hipStream_t stream);

bool bwd_mfma_supported(const Problem& pr, const Groups& G);
size_t bwd_mfma_workspace_bytes(const Problem& pr, const Groups& G);
hipError_t launch_bwd_mfma(const Problem& pr, const Groups& G, const void* q, const void* k,
                           const void* v, const void* o, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv, void* workspace, hipStream_t stream);

// dQ kernel of the MFMA backward at head dims 64 and 128 (attn_bwd_dq.hip),
// for the configurations the dispatch in attn_bwd_mfma.hip uses.  A wave
// holds whole rows; the kernel also forms Delta = rowsum(dO*O) of its rows
// and writes it with LSE*log2(e) (+inf where LSE = -inf) to `delta` and
// `lse2`.
template <int D, int BN, int NW, int NS>
hipError_t launch_bwd_dq(const Problem& pr, const Groups& G, const GroupBlocks& gb, int HG, int64_t nwg,
                         const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                         const uint16_t* o, const float* lse, float* delta, float* lse2, uint16_t* dq,
                         hipStream_t stream);

// dQ kernel at head dim 256, one wave per SIMD (attn_bwd_dq_wide.hip); forms
// Delta and LSE*log2(e) like the DS == 1 configurations above.
hipError_t launch_bwd_dq_wide(const Problem& pr, const Groups& G, const GroupBlocks& gb, int HG, int64_t nwg,
                              const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                              const uint16_t* o, const float* lse, float* delta, float* lse2, uint16_t* dq,
                              hipStream_t stream);

// Scalar backward: delta[h][t] = sum_d dO[t,h,d] * O[t,h,d] in fp32 (0 on
// rows with no visible key) for all pr.Tld rows.
hipError_t launch_bwd_delta(const Problem& pr, int dtype, const void* o, const void* dout,
                            const float* lse, float* delta, hipStream_t stream);

}  // namespace dualkv
