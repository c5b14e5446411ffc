// Scalar (non-MFMA) shared-prompt attention: one wavefront per output row.
//
// This path computes in fp32 for both element types and accepts any head
// dim 1..512.  It serves the fp32 dtype (whose tolerance needs true fp32
// products) and head dims without an MFMA tiling.  Visibility follows
// "DualKV: Shared-Prompt Flash Attention ..." (arXiv 2605.15422), Abstract:
// a prompt query sees the prompt causally; a response query sees the whole
// prompt and then its own response causally, one softmax over both ranges.
//
// Forward: online softmax over 64-key chunks (lane = key for the scores,
// lane = head-dim slice for the accumulator).  Backward: dQ per query row
// and dK/dV per key row, each summed by a single wavefront in a fixed
// order (query heads of the group ascending, prompt queries first, then
// responses ascending), so results are deterministic without atomics.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace dualkv {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxD = 512;
constexpr int kDpl = kMaxD / 64;   // head-dim slots per lane

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Key rows visible to packed query row t: prompt rows [a0, a1) then own
// response rows [b0, b1) (both in ascending logical position).
struct KeyRanges {
  int a0, a1, b0, b1;
  bool valid;
};

__device__ KeyRanges keys_of_query(const Problem& pr, int t) {
  KeyRanges kr{0, 0, 0, 0, false};
  if (t < pr.P) {
    kr.valid = true;
    kr.a0 = pr.W > 0 ? max(0, t - pr.W + 1) : 0;
    kr.a1 = t + 1;
    return kr;
  }
  int rel = t - pr.P, n = rel / pr.R, r = rel - n * pr.R;
  if (r >= resp_valid(pr, n)) return kr;
  kr.valid = true;
  int qpos = pr.P + r;
  int lo = pr.W > 0 ? max(0, qpos - pr.W + 1) : 0;   // lowest visible position
  kr.a0 = min(lo, pr.P);
  kr.a1 = pr.P;
  int base = pr.P + n * pr.R;
  kr.b0 = base + max(0, lo - pr.P);
  kr.b1 = base + r + 1;
  return kr;
}

template <typename T>
__global__ void __launch_bounds__(256) fwd_scalar_kernel(Problem pr, const T* __restrict__ q,
                                                         const T* __restrict__ k,
                                                         const T* __restrict__ v, T* __restrict__ o,
                                                         float* __restrict__ lse) {
  __shared__ float qs[kWaves][kMaxD];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
  const bool active = item < (int64_t)pr.T * pr.Hq;
  const int t = active ? (int)(item / pr.Hq) : 0;
  const int h = active ? (int)(item % pr.Hq) : 0;
  const int c = h / pr.g, D = pr.D;
  const int64_t qoff = ((int64_t)t * pr.Hq + h) * D;
  for (int d = lane; d < D; d += 64) qs[wave][d] = active ? Elem<T>::load(q + qoff + d) : 0.f;
  __syncthreads();
  if (!active) return;
  KeyRanges kr = keys_of_query(pr, t);
  float m = -INFINITY, l = 0.f, acc[kDpl];
#pragma unroll
  for (int i = 0; i < kDpl; ++i) acc[i] = 0.f;
  for (int part = 0; part < 2 && kr.valid; ++part) {
    const int s0 = part == 0 ? kr.a0 : kr.b0, s1 = part == 0 ? kr.a1 : kr.b1;
    for (int base = s0; base < s1; base += 64) {
      const int j = base + lane;
      float s = -INFINITY;
      if (j < s1) {
        const T* kp = k + ((int64_t)j * pr.Hkv + c) * D;
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(qs[wave][d], Elem<T>::load(kp + d), dot);
        s = dot * pr.scale;
      }
      const float mn = fmaxf(m, wave_max(s));
      const float alpha = expf(m - mn);
      const float p = j < s1 ? expf(s - mn) : 0.f;
      l = l * alpha + wave_sum(p);
#pragma unroll
      for (int i = 0; i < kDpl; ++i) acc[i] *= alpha;
      const int cnt = min(64, s1 - base);
      for (int jj = 0; jj < cnt; ++jj) {
        const float pj = __shfl(p, jj, 64);
        const T* vp = v + ((int64_t)(base + jj) * pr.Hkv + c) * D;
#pragma unroll
        for (int i = 0; i < kDpl; ++i) {
          const int d = lane + 64 * i;
          if (d < D) acc[i] = fmaf(pj, Elem<T>::load(vp + d), acc[i]);
        }
      }
      m = mn;
    }
  }
  const bool has = kr.valid && l > 0.f;
  const float inv = has ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < kDpl; ++i) {
    const int d = lane + 64 * i;
    if (d < D) Elem<T>::store(o + qoff + d, acc[i] * inv);
  }
  if (lane == 0) lse[(int64_t)h * pr.Tld + t] = has ? m + logf(l) : -INFINITY;
}

template <typename T>
__global__ void __launch_bounds__(256) delta_kernel(Problem pr, const T* __restrict__ o,
                                                    const T* __restrict__ dout,
                                                    const float* __restrict__ lse,
                                                    float* __restrict__ delta) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
  if (item >= (int64_t)pr.Tld * pr.Hq) return;        // every row of the launch
  const int t = (int)(item / pr.Hq), h = (int)(item % pr.Hq);
  const int64_t off = ((int64_t)t * pr.Hq + h) * pr.D;
  float s = 0.f;
  for (int d = lane; d < pr.D; d += 64) s = fmaf(Elem<T>::load(dout + off + d), Elem<T>::load(o + off + d), s);
  s = wave_sum(s);
  const float L = lse[(int64_t)h * pr.Tld + t];
  if (lane == 0) delta[(int64_t)h * pr.Tld + t] = L == -INFINITY ? 0.f : s;
}

template <typename T>
__global__ void __launch_bounds__(256) dq_scalar_kernel(Problem pr, const T* __restrict__ q,
                                                        const T* __restrict__ k,
                                                        const T* __restrict__ v,
                                                        const T* __restrict__ dout,
                                                        const float* __restrict__ lse,
                                                        const float* __restrict__ delta,
                                                        T* __restrict__ dq) {
  __shared__ float qs[kWaves][kMaxD];
  __shared__ float dos[kWaves][kMaxD];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
  const bool active = item < (int64_t)pr.T * pr.Hq;
  const int t = active ? (int)(item / pr.Hq) : 0;
  const int h = active ? (int)(item % pr.Hq) : 0;
  const int c = h / pr.g, D = pr.D;
  const int64_t qoff = ((int64_t)t * pr.Hq + h) * D;
  for (int d = lane; d < D; d += 64) {
    qs[wave][d] = active ? Elem<T>::load(q + qoff + d) : 0.f;
    dos[wave][d] = active ? Elem<T>::load(dout + qoff + d) : 0.f;
  }
  __syncthreads();
  if (!active) return;
  KeyRanges kr = keys_of_query(pr, t);
  const float L = lse[(int64_t)h * pr.Tld + t];
  const float Dl = delta[(int64_t)h * pr.Tld + t];
  float acc[kDpl];
#pragma unroll
  for (int i = 0; i < kDpl; ++i) acc[i] = 0.f;
  const bool live = kr.valid && L != -INFINITY;
  for (int part = 0; part < 2 && live; ++part) {
    const int s0 = part == 0 ? kr.a0 : kr.b0, s1 = part == 0 ? kr.a1 : kr.b1;
    for (int base = s0; base < s1; base += 64) {
      const int j = base + lane;
      float ds = 0.f;
      if (j < s1) {
        const T* kp = k + ((int64_t)j * pr.Hkv + c) * D;
        const T* vp = v + ((int64_t)j * pr.Hkv + c) * D;
        float sdot = 0.f, pdot = 0.f;
        for (int d = 0; d < D; ++d) {
          sdot = fmaf(qs[wave][d], Elem<T>::load(kp + d), sdot);
          pdot = fmaf(dos[wave][d], Elem<T>::load(vp + d), pdot);
        }
        const float p = expf(sdot * pr.scale - L);
        ds = p * (pdot - Dl);
      }
      const int cnt = min(64, s1 - base);
      for (int jj = 0; jj < cnt; ++jj) {
        const float dsj = __shfl(ds, jj, 64);
        const T* kp = k + ((int64_t)(base + jj) * pr.Hkv + c) * D;
#pragma unroll
        for (int i = 0; i < kDpl; ++i) {
          const int d = lane + 64 * i;
          if (d < D) acc[i] = fmaf(dsj, Elem<T>::load(kp + d), acc[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kDpl; ++i) {
    const int d = lane + 64 * i;
    if (d < D) Elem<T>::store(dq + qoff + d, acc[i] * pr.scale);
  }
}

template <typename T>
__global__ void __launch_bounds__(256) dkdv_scalar_kernel(Problem pr, const T* __restrict__ q,
                                                          const T* __restrict__ k,
                                                          const T* __restrict__ v,
                                                          const T* __restrict__ dout,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ delta,
                                                          T* __restrict__ dk, T* __restrict__ dv) {
  __shared__ float ks[kWaves][kMaxD];
  __shared__ float vs[kWaves][kMaxD];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
  const bool active = item < (int64_t)pr.T * pr.Hkv;
  const int j = active ? (int)(item / pr.Hkv) : 0;
  const int c = active ? (int)(item % pr.Hkv) : 0;
  const int D = pr.D;
  const int64_t koff = ((int64_t)j * pr.Hkv + c) * D;
  for (int d = lane; d < D; d += 64) {
    ks[wave][d] = active ? Elem<T>::load(k + koff + d) : 0.f;
    vs[wave][d] = active ? Elem<T>::load(v + koff + d) : 0.f;
  }
  __syncthreads();
  if (!active) return;
  // Which queries see key row j: for a prompt key (position j) the prompt
  // queries j.. and the first rows of every response (all of them without a
  // window); for a response key only the later rows of its own response.
  bool kvalid;
  int kpos, own_n = -1;
  if (j < pr.P) {
    kvalid = true;
    kpos = j;
  } else {
    int rel = j - pr.P, n = rel / pr.R, r = rel - n * pr.R;
    kvalid = r < resp_valid(pr, n);
    kpos = pr.P + r;
    own_n = n;
  }
  float akk[kDpl], avv[kDpl];
#pragma unroll
  for (int i = 0; i < kDpl; ++i) akk[i] = avv[i] = 0.f;
  for (int h = c * pr.g; h < (c + 1) * pr.g && kvalid; ++h) {
    const int n_first = own_n >= 0 ? own_n : -1;
    const int n_last = own_n >= 0 ? own_n : pr.N - 1;
    for (int seg = n_first; seg <= n_last; ++seg) {
      int s0, s1;
      if (seg < 0) {  // prompt queries
        s0 = j;
        s1 = pr.W > 0 ? min(pr.P, j + pr.W) : pr.P;
      } else {
        const int Lv = resp_valid(pr, seg);
        const int rlo = max(0, kpos - pr.P);
        int rhi = Lv;
        if (pr.W > 0) rhi = min(rhi, max(0, kpos + pr.W - pr.P));
        s0 = pr.P + seg * pr.R + rlo;
        s1 = pr.P + seg * pr.R + max(rlo, rhi);
      }
      for (int base = s0; base < s1; base += 64) {
        const int i = base + lane;
        float p = 0.f, ds = 0.f;
        if (i < s1) {
          const T* qp = q + ((int64_t)i * pr.Hq + h) * D;
          const T* dp = dout + ((int64_t)i * pr.Hq + h) * D;
          float sdot = 0.f, pdot = 0.f;
          for (int d = 0; d < D; ++d) {
            sdot = fmaf(Elem<T>::load(qp + d), ks[wave][d], sdot);
            pdot = fmaf(Elem<T>::load(dp + d), vs[wave][d], pdot);
          }
          p = expf(sdot * pr.scale - lse[(int64_t)h * pr.Tld + i]);
          ds = p * (pdot - delta[(int64_t)h * pr.Tld + i]);
        }
        const int cnt = min(64, s1 - base);
        for (int ii = 0; ii < cnt; ++ii) {
          const float pi = __shfl(p, ii, 64), dsi = __shfl(ds, ii, 64);
          const T* qp = q + ((int64_t)(base + ii) * pr.Hq + h) * D;
          const T* dp = dout + ((int64_t)(base + ii) * pr.Hq + h) * D;
#pragma unroll
          for (int x = 0; x < kDpl; ++x) {
            const int d = lane + 64 * x;
            if (d < D) {
              avv[x] = fmaf(pi, Elem<T>::load(dp + d), avv[x]);
              akk[x] = fmaf(dsi, Elem<T>::load(qp + d), akk[x]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int x = 0; x < kDpl; ++x) {
    const int d = lane + 64 * x;
    if (d < D) {
      Elem<T>::store(dk + koff + d, akk[x] * pr.scale);
      Elem<T>::store(dv + koff + d, avv[x]);
    }
  }
}

unsigned blocks_for(int64_t items) { return (unsigned)((items + kWaves - 1) / kWaves); }

// Byte offset of packed row `row` in a [rows, H, D] tensor.
int64_t row_bytes_at(int64_t row, int H, int D, int dtype) {
  return row * H * D * (dtype == DUALKV_F32 ? 4 : 2);
}
template <typename T>
T* at(T* p, int64_t bytes) {
  using B = typename std::conditional<std::is_const<T>::value, const char, char>::type;
  return reinterpret_cast<T*>(reinterpret_cast<B*>(p) + bytes);
}

}  // namespace

// One launch per prompt group (the scalar path is the exactness path, not
// a fast one); each group's tensors and [H, Tld] rows are offset to its row 0.
hipError_t launch_fwd_scalar(const Problem& pr, const Groups& G, int dtype, const void* q,
                             const void* k, const void* v, void* o, float* lse, hipStream_t stream) {
  for (int gi = 0; gi < G.n; ++gi) {
    const Problem gp = group_problem(pr, G, gi);
    if (gp.T == 0) continue;
    const int64_t r0 = G.row0[gi];
    const void* qg = at(q, row_bytes_at(r0, pr.Hq, pr.D, dtype));
    const void* kg = at(k, row_bytes_at(r0, pr.Hkv, pr.D, dtype));
    const void* vg = at(v, row_bytes_at(r0, pr.Hkv, pr.D, dtype));
    void* og = at(o, row_bytes_at(r0, pr.Hq, pr.D, dtype));
    float* lg = lse + r0;
    const dim3 grid(blocks_for((int64_t)gp.T * pr.Hq)), block(64 * kWaves);
    hipError_t e;
    if (dtype == DUALKV_F32)
      e = launch("fwd_scalar", fwd_scalar_kernel<float>, grid, block, 0, stream, gp, (const float*)qg,
                 (const float*)kg, (const float*)vg, (float*)og, lg);
    else
      e = launch("fwd_scalar", fwd_scalar_kernel<uint16_t>, grid, block, 0, stream, gp, (const uint16_t*)qg,
                 (const uint16_t*)kg, (const uint16_t*)vg, (uint16_t*)og, lg);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_bwd_delta(const Problem& pr, int dtype, const void* o, const void* dout,
                            const float* lse, float* delta, hipStream_t stream) {
  const dim3 grid(blocks_for((int64_t)pr.Tld * pr.Hq)), block(64 * kWaves);
  if (dtype == DUALKV_F32)
    return launch("bwd_delta", delta_kernel<float>, grid, block, 0, stream, pr, (const float*)o,
                  (const float*)dout, lse, delta);
  return launch("bwd_delta", delta_kernel<uint16_t>, grid, block, 0, stream, pr, (const uint16_t*)o,
                (const uint16_t*)dout, lse, delta);
}

hipError_t launch_bwd_scalar(const Problem& pr, const Groups& G, int dtype, const void* q,
                             const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, float* delta,
                             hipStream_t stream) {
  hipError_t e = launch_bwd_delta(pr, dtype, o, dout, lse, delta, stream);
  if (e != hipSuccess) return e;
  const dim3 block(64 * kWaves);
  for (int gi = 0; gi < G.n; ++gi) {
    const Problem gp = group_problem(pr, G, gi);
    if (gp.T == 0) continue;
    const int64_t r0 = G.row0[gi];
    const int64_t bq = row_bytes_at(r0, pr.Hq, pr.D, dtype), bk = row_bytes_at(r0, pr.Hkv, pr.D, dtype);
    const dim3 gq(blocks_for((int64_t)gp.T * pr.Hq)), gk(blocks_for((int64_t)gp.T * pr.Hkv));
    const float* lg = lse + r0;
    const float* dg = delta + r0;
    if (dtype == DUALKV_F32) {
      e = launch("bwd_dq_scalar", dq_scalar_kernel<float>, gq, block, 0, stream, gp, at((const float*)q, bq),
                 at((const float*)k, bk), at((const float*)v, bk), at((const float*)dout, bq), lg, dg,
                 at((float*)dq, bq));
      if (e != hipSuccess) return e;
      e = launch("bwd_dkdv_scalar", dkdv_scalar_kernel<float>, gk, block, 0, stream, gp, at((const float*)q, bq),
                 at((const float*)k, bk), at((const float*)v, bk), at((const float*)dout, bq), lg, dg,
                 at((float*)dk, bk), at((float*)dv, bk));
    } else {
      e = launch("bwd_dq_scalar", dq_scalar_kernel<uint16_t>, gq, block, 0, stream, gp,
                 at((const uint16_t*)q, bq), at((const uint16_t*)k, bk), at((const uint16_t*)v, bk),
                 at((const uint16_t*)dout, bq), lg, dg, at((uint16_t*)dq, bq));
      if (e != hipSuccess) return e;
      e = launch("bwd_dkdv_scalar", dkdv_scalar_kernel<uint16_t>, gk, block, 0, stream, gp,
                 at((const uint16_t*)q, bq), at((const uint16_t*)k, bk), at((const uint16_t*)v, bk),
                 at((const uint16_t*)dout, bq), lg, dg, at((uint16_t*)dk, bk), at((uint16_t*)dv, bk));
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dualkv
